#!/usr/bin/env python3
"""Benchmark of the MI355X attention forward kernel.

Prints one JSON line: attention-forward TFLOP/s on the causal grouped-query workload
(B=1, Hq=32, Hkv=4, Sq=Skv=8192, D=128, bf16), its fraction of the MI355X dense bf16
MFMA peak, and the fp64 CPU oracle timed on a bounded sample of the same workload.

FLOPs are counted as 4*B*Hq*Sq*Skv*D, halved when causal.  Inputs are resident in HBM
before the timed region; each step is one call of the library's fa_fwd on torch's
current stream, timed with HIP events recorded on that stream: the K timed steps run back
to back between two events (value, ms_per_step), then K more with an event pair around each
launch give the per-launch durations (kernel_us, roofline.achieved).

Warm-up: W untimed steps, then more untimed steps until at least MIN_WARMUP_S seconds of
warm-up have passed.  Coming out of idle the GPU needs some tens of milliseconds to reach
its working clock (the first ~30 launches of the headline kernel run up to 30% slower),
so a fixed small W would time the clock ramp rather than the kernel.  The extra steps are
reported as "warmup_extra_steps".

--splitkv times fa_fwd_splitkv (fa_fwd_splitkv_fp8 for an fp8 workload; the library's split
count, workspace allocated before the timed region) instead; decoding workloads (one query
row) are reported in GB/s against the HBM roofline, since reading K and V bounds them.

--cold writes 512 MiB (twice the last-level cache) before each launch, outside the events
that time it, so every launch starts with cold caches.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--splitkv]
                       [--backward] [--cold] [--sweep] [--all]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MI355X dense bf16 MFMA peak (causal, D=128)"
HEADLINE = "gqa8_causal_s8192_d128_bf16"
# MI355X dense bf16/fp16 MFMA peak: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU; fp8 twice that.
PEAK_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
PEAK_FP8_TFLOPS = 2 * PEAK_TFLOPS
# fp8 Q/K workloads: half the FLOPs (Q K^T) at the fp8 peak, half (P V) at the bf16 one.
PEAK_FP8QK_TFLOPS = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_TFLOPS)
METRIC_BWD = "attention bwd TFLOP/s (2.5x the forward FLOPs: five matrix products), bf16/fp16"
METRIC_FP8 = "attention fwd TFLOP/s, fp8 E4M3 Q/K (Q K^T on the fp8 MFMA), fp16/bf16 P V"
METRIC_FP8QKV = ("attention fwd TFLOP/s, fp8 E4M3 Q/K/V (Q K^T on the fp8 MFMA; V widened to "
                 "bf16/fp16 for P V)")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_traffic.json")
MIN_WARMUP_S = 0.3
COLD_FLUSH_BYTES = 512 << 20
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
KERNEL_SOURCES = [os.path.join(ROOT, "attention_fa_fwd_amd", "csrc", f)
                  for f in ("fa_fwd_kernel.hpp", "fa_fwd.hip")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def literal_flops(w):
    """4*B*Hq*Sq*Skv*D, halved when causal; a sliding window counts its visible pairs."""
    if w.get("window", 0):
        return exact_flops(w)
    f = 4.0 * w["B"] * w["Hq"] * w["Sq"] * w["Skv"] * w["D"]
    return f / 2 if w["causal"] else f


def exact_flops(w):
    """4*D per visible (query, key) pair."""
    Sq, Skv, pos = w["Sq"], w["Skv"], w["input_pos"]
    W = w.get("window", 0)
    if W:
        import numpy as np

        i = np.arange(Sq, dtype=np.int64) + pos
        hi = np.minimum(i, Skv - 1)
        lo = np.maximum(i - W + 1, 0)
        pairs = int(np.maximum(hi - lo + 1, 0).sum())
    elif not w["causal"]:
        pairs = Sq * Skv
    else:
        pairs = 0
        # visible keys of row i: min(Skv, pos + i + 1)
        full_from = max(0, Skv - pos - 1)  # rows i >= full_from see every key
        n_part = min(Sq, full_from)
        pairs += n_part * (pos + 1) + n_part * (n_part - 1) // 2
        pairs += (Sq - n_part) * Skv
    return 4.0 * w["D"] * w["B"] * w["Hq"] * pairs


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_bytes(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if the
    kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    e = t.get("workloads", {}).get(workload)
    if not e:
        return None
    return e.get("hbm_bytes_per_launch")


def algorithmic_bytes(w, fp8=False):
    """q, k, v read once; out and lse written once (q and k one byte per element with fp8,
    v too for an fp8 Q/K/V workload)."""
    qk = 1 if fp8 else 2
    vb = 1 if w.get("fp8v") else 2
    q_o = w["B"] * w["Hq"] * w["Sq"] * w["D"] * (qk + 2)
    k_v = w["B"] * w["Hkv"] * w["Skv"] * w["D"] * (qk + vb)
    return q_o + k_v + w["B"] * w["Hq"] * w["Sq"] * 4


def workload(name):
    """(shape dict, is fp8) of a named workload."""
    from attention_fa_fwd_amd.inputs import FP8_WORKLOADS, SWEEP_WORKLOADS, WORKLOADS

    if name in FP8_WORKLOADS:
        return FP8_WORKLOADS[name], True
    if name in SWEEP_WORKLOADS:
        return SWEEP_WORKLOADS[name], False
    return WORKLOADS[name], False


def time_gpu(name, steps, warmup, config=-1, splitkv=False, backward=False, cold=False):
    import torch

    import attention_fa_fwd_amd as fa
    from attention_fa_fwd_amd.inputs import make_fp8_workload, make_workload

    w, fp8 = workload(name)
    fp8v = fp8 and w.get("fp8v", False)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if fp8:
        q, k, v, kw = make_fp8_workload(name, seed=0)
    else:
        q, k, v, kw = make_workload(name, seed=0)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    out_dtype = {"bf16": torch.bfloat16, "fp16": torch.float16}[w["dtype"]]
    out = torch.empty(q.shape, dtype=out_dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    splits = 1
    if backward:
        fa.fa_fwd_into(q, k, v, out, lse, scale=kw["scale"], causal=kw["causal"],
                       input_pos=kw["input_pos"], window=kw["window"], stream=sp)
        g = torch.Generator(device="cpu")
        g.manual_seed(1)
        dout = torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype).to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(max(16, fa.bwd_workspace_size(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"],
                                                      w["D"], kw["causal"])),
                         dtype=torch.uint8, device=dev)

        def step():
            fa.fa_bwd_into(q, k, v, out, lse, dout, dq, dk, dv, ws, scale=kw["scale"],
                           causal=kw["causal"], input_pos=kw["input_pos"], window=kw["window"],
                           stream=sp)
    elif fp8v and splitkv:
        splits = fa.splitkv_num_splits_fp8qkv(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"],
                                              w["causal"], w["input_pos"], out_dtype, config,
                                              kw["window"])
        nbytes = fa.splitkv_workspace_size(w["B"], w["Hq"], w["Sq"], w["D"], splits)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None

        def step():
            fa.fa_fwd_splitkv_fp8qkv_into(q, k, v, out, lse, ws, kw["q_descale"], kw["k_descale"],
                                          kw["v_descale"], num_splits=splits, scale=kw["scale"],
                                          causal=kw["causal"], input_pos=kw["input_pos"],
                                          window=kw["window"], config=config, stream=sp)
    elif fp8v:
        def step():
            fa.fa_fwd_fp8qkv_into(q, k, v, out, lse, kw["q_descale"], kw["k_descale"],
                                  kw["v_descale"], scale=kw["scale"], causal=kw["causal"],
                                  input_pos=kw["input_pos"], window=kw["window"], config=config,
                                  stream=sp)
    elif fp8 and splitkv:
        splits = fa.splitkv_num_splits_fp8(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"],
                                           w["causal"], w["input_pos"], v.dtype, config,
                                           kw["window"])
        nbytes = fa.splitkv_workspace_size(w["B"], w["Hq"], w["Sq"], w["D"], splits)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None

        def step():
            fa.fa_fwd_splitkv_fp8_into(q, k, v, out, lse, ws, kw["q_descale"], kw["k_descale"],
                                       num_splits=splits, scale=kw["scale"], causal=kw["causal"],
                                       input_pos=kw["input_pos"], window=kw["window"],
                                       config=config, stream=sp)
    elif fp8:
        def step():
            fa.fa_fwd_fp8_into(q, k, v, out, lse, kw["q_descale"], kw["k_descale"],
                               scale=kw["scale"], causal=kw["causal"], input_pos=kw["input_pos"],
                               window=kw["window"], config=config, stream=sp)
    elif splitkv:
        splits = fa.splitkv_num_splits(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"],
                                       w["causal"], w["input_pos"], q.dtype, config,
                                       kw["window"])
        nbytes = fa.splitkv_workspace_size(w["B"], w["Hq"], w["Sq"], w["D"], splits)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None

        def step():
            fa.fa_fwd_splitkv_into(q, k, v, out, lse, ws, num_splits=splits, scale=kw["scale"],
                                   causal=kw["causal"], input_pos=kw["input_pos"], config=config,
                                   stream=sp, window=kw["window"])
    else:
        # Arguments checked and marshalled once; each step is one C call (a few microseconds
        # of host time, against about ten through fa_fwd_into, which short workloads feel).
        step = fa.fa_fwd_prepared(q, k, v, out, lse, scale=kw["scale"], causal=kw["causal"],
                                  input_pos=kw["input_pos"], config=config, stream=sp,
                                  window=kw["window"])

    t_warm = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    extra = 0
    while time.perf_counter() - t_warm < MIN_WARMUP_S:
        for _ in range(10):
            step()
        extra += 10
        torch.cuda.synchronize()
    if cold:
        # Cold caches: write COLD_FLUSH_BYTES (twice the 256 MB last-level cache) before each
        # launch, outside the events that time it.
        flush = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device=dev)
        ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            flush.fill_(i & 255)
            ev0[i].record(stream)
            step()
            ev1[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = sorted(ev0[i].elapsed_time(ev1[i]) for i in range(steps))
        total_ms = sum(per)
    else:
        # Throughput: K steps back to back between two events (nothing else on the stream).
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total_ms = e0.elapsed_time(e1)
        # Per-launch durations: K more steps with an event between every two launches (the
        # events add a gap of a few microseconds per launch, which the throughput run has not).
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(steps):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))  # ms per launch
    if config >= 0:
        cfg = config
    elif fp8:
        cfg = fa.select_config_fp8(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["D"], w["causal"], out_dtype)
        if fp8v:   # the fp8 Q/K/V table entry of the same shape
            cfg = fa.config_names().index(fa.config_names()[cfg].replace("_fp8qk_", "_fp8qkv_"))
    else:
        cfg = fa.select_config(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"], w["causal"],
                               w["input_pos"], q.dtype)
    kernel = "fa_bwd (dot, dK/dV, dQ)" if backward else fa.config_names()[cfg]
    if splitkv and splits > 1 and "_KS2_" in kernel:
        kernel = kernel.replace("_KS2_", "_")   # split-KV runs the one-key-part twin
    return dict(total_ms=total_ms, wall_s=wall, per_ms=per, kernel=kernel,
                warmup_extra=extra, splits=splits)


def _blas_threads():
    """Threads of the BLAS pool NumPy's matmul runs on (threadpoolctl), or None."""
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else None
    except Exception:  # pragma: no cover - threadpoolctl missing
        return None


def cpu_baseline(name, min_s=10.0, backward=False, unit="TFLOP/s"):
    """The fp64 oracle of the timed path (forward, fp8 forward or backward) on whole GQA
    groups (one K/V head and its query heads) of the workload, one group after another until
    at least ``min_s`` seconds of CPU work have run or the workload is exhausted (a bounded
    sample; every group has the same shape).  BLAS runs on every core the process may use
    (os.sched_getaffinity); ``cores`` is the size of the BLAS pool that ran, next to that
    count.  The rate is in the bench line's own unit: TFLOP/s under the same FLOP rule, or
    for a decoding line GB/s of the same algorithmic bytes.  The smallest workload also gets
    the single-core pure-Python form."""
    import numpy as np
    import torch

    import oracle
    from attention_fa_fwd_amd.inputs import make_fp8_workload, make_workload

    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=affinity, user_api="blas")
    except Exception:  # pragma: no cover - threadpoolctl missing
        limiter = None
    threads = _blas_threads() or affinity
    w, fp8 = workload(name)
    fp8v = fp8 and w.get("fp8v", False)
    if fp8:
        q, k, v, kw = make_fp8_workload(name, seed=0)
    else:
        q, k, v, kw = make_workload(name, seed=0)
    codes = lambda t: t.view(torch.uint8).numpy()
    G = w["Hq"] // w["Hkv"]
    groups = [(b, g) for b in range(w["B"]) for g in range(w["Hkv"])]
    if backward:
        gen = torch.Generator(device="cpu")
        gen.manual_seed(1)
        dout = torch.randn(q.shape, generator=gen, dtype=torch.float32).to(q.dtype)
    done, dt = 0, 0.0
    for b, g in groups:
        sl_q, sl_k = (slice(b, b + 1), slice(g * G, (g + 1) * G)), (slice(b, b + 1), slice(g, g + 1))
        t0 = time.perf_counter()
        if fp8:
            oracle.attention_fp8_blocked(codes(q[sl_q]), codes(k[sl_k]),
                                         codes(v[sl_k]) if fp8v else v[sl_k].double().numpy(),
                                         kw["scale"], kw["q_descale"], kw["k_descale"], kw["causal"],
                                         kw["input_pos"], window=kw["window"],
                                         v_descale=kw.get("v_descale"))
        elif backward:
            oracle.attention_backward_blocked(q[sl_q].double().numpy(), k[sl_k].double().numpy(),
                                              v[sl_k].double().numpy(), dout[sl_q].double().numpy(),
                                              kw["scale"], kw["causal"], kw["input_pos"],
                                              window=kw["window"])
        else:
            oracle.attention_blocked(q[sl_q].double().numpy(), k[sl_k].double().numpy(),
                                     v[sl_k].double().numpy(), kw["scale"], kw["causal"],
                                     kw["input_pos"], window=kw["window"])
        dt += time.perf_counter() - t0
        done += 1
        if dt >= min_s:
            break
    if limiter is not None:
        limiter.restore_original_limits()
    ws = dict(w, B=1, Hq=G, Hkv=1)
    form = ("fp8 forward" if fp8 else "backward" if backward else "forward") + " oracle (NumPy, fp64)"
    if unit == "GB/s":
        value, rule = done * algorithmic_bytes(ws, fp8) / dt / 1e9, "same algorithmic byte count"
    else:
        value = done * literal_flops(ws) * (2.5 if backward else 1.0) / dt / 1e12
        rule = "same FLOP count rule"
    out = dict(value=value, unit=unit, cores=int(threads), kind="oracle",
               sample=f"{form}: {done} of the {len(groups)} GQA groups (one K/V head and its {G} "
                      f"query heads each) of {name}; {dt:.1f} s wall; {rule}",
               wall_s=round(dt, 3), affinity_cores=affinity)
    if w["B"] * w["Hq"] * w["Sq"] * w["Skv"] <= 1 << 16 and not fp8 and not backward:
        # the pure-Python loops, one core, on the whole (tiny) workload
        t0 = time.perf_counter()
        oracle.attention_naive(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                               kw["scale"], kw["causal"], kw["input_pos"], window=kw["window"])
        t1 = time.perf_counter() - t0
        out["naive_single_core"] = dict(value=literal_flops(w) / t1 / 1e12, unit="TFLOP/s",
                                        cores=1, wall_s=round(t1, 3),
                                        sample=f"pure-Python loops over all of {name}")
    return out


def bench_line(name, steps, warmup, config=-1, with_cpu=True, splitkv=False, backward=False,
               cold=False):
    w, fp8 = workload(name)
    log(f"workload {name}: {w}")
    r = time_gpu(name, steps, warmup, config, splitkv, backward, cold)
    ms_step = r["total_ms"] / steps
    flops = literal_flops(w) * (2.5 if backward else 1.0)
    value = flops / (ms_step * 1e-3) / 1e12
    mean_kernel_ms = sum(r["per_ms"]) / len(r["per_ms"])
    med = r["per_ms"][len(r["per_ms"]) // 2]
    p95 = r["per_ms"][min(len(r["per_ms"]) - 1, int(math.ceil(0.95 * len(r["per_ms"]))) - 1)]
    fp8v = fp8 and w.get("fp8v", False)
    path = ("fa_bwd" if backward else
            f"fa_fwd_splitkv_fp8qkv ({r['splits']} splits)" if fp8v and splitkv else
            "fa_fwd_fp8qkv" if fp8v else
            f"fa_fwd_splitkv_fp8 ({r['splits']} splits)" if fp8 and splitkv else
            "fa_fwd_fp8" if fp8 else
            f"fa_fwd_splitkv ({r['splits']} splits)" if splitkv else "fa_fwd")
    log(f"{path} kernel {r['kernel']}: mean {mean_kernel_ms * 1e3:.1f} us, median {med * 1e3:.1f} us, "
        f"p95 {p95 * 1e3:.1f} us, min {r['per_ms'][0] * 1e3:.1f} us, "
        f"{r['warmup_extra']} extra warm-up steps")
    decode = w["Sq"] <= 16 and not backward
    if decode:
        # Reading K and V bounds a decoding step: GB/s of algorithmic bytes per call, over the
        # throughput run (value) and over the mean per-call duration (roofline).
        nbytes = algorithmic_bytes(w, fp8)
        gbs = nbytes / (mean_kernel_ms * 1e-3) / 1e9
        metric, value, unit = ("attention decode GB/s of algorithmic HBM bytes",
                               nbytes / (ms_step * 1e-3) / 1e9, "GB/s")
        # Counted bytes of the attention kernel (the merge kernel's are not included).
        traffic = None if cold else traffic_bytes(name + ("/splitkv" if splitkv else ""))
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        achieved = flops / (mean_kernel_ms * 1e-3) / 1e12
        metric, unit = (METRIC_BWD if backward else METRIC_FP8QKV if fp8v else
                        METRIC_FP8 if fp8 else METRIC), "TFLOP/s"
        peak = PEAK_FP8QK_TFLOPS if fp8 else PEAK_TFLOPS
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": None if (splitkv or backward or cold) else traffic_bytes(name)}
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "warmup_extra_steps": r["warmup_extra"],
        "warmup_total_steps": warmup + r["warmup_extra"],
        "warmup_rule": f"{warmup} steps, then more until {MIN_WARMUP_S} s of warm-up (clock ramp)",
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"fp8e4m3 q/k/v, {w['dtype']} out" if fp8v else
                  f"fp8e4m3 q/k, {w['dtype']} v" if fp8 else w["dtype"]),
        "data": ("synthetic: seeded N(0,1) q, k, v quantised per tensor to fp8 e4m3" if fp8v else
                 "synthetic: seeded N(0,1) q, k quantised per tensor to fp8 e4m3, v rounded to "
                 "the storage dtype" if fp8 else
                 "synthetic: seeded N(0,1) q, k, v rounded to the storage dtype"),
        "config": {"workload": name, "B": w["B"], "Hq": w["Hq"], "Hkv": w["Hkv"], "Sq": w["Sq"],
                   "Skv": w["Skv"], "D": w["D"], "causal": w["causal"],
                   "input_pos": w["input_pos"], "window": w.get("window", 0),
                   "kernel": r["kernel"], "path": path,
                   "caches": (f"cold: {COLD_FLUSH_BYTES >> 20} MiB written before each launch, "
                              "outside its events") if cold else "warm: launches back to back",
                   "timing": ("each launch between its own events (value and kernel_us)" if cold else
                              "value and ms_per_step: the K steps back to back between two events; "
                              "kernel_us and roofline.achieved: K more steps, an event pair around "
                              "each launch"),
                   "parallelism": "single GPU"},
        "kernel_us": {"mean": round(mean_kernel_ms * 1e3, 2), "median": round(med * 1e3, 2),
                      "p95": round(p95 * 1e3, 2), "min": round(r["per_ms"][0] * 1e3, 2)},
        "roofline": roofline,
    }
    if not decode:
        line["pct_of_peak"] = round(100.0 * value / (PEAK_FP8QK_TFLOPS if fp8 else PEAK_TFLOPS), 2)
        line["tflops_exact_pairs"] = round(exact_flops(w) * (2.5 if backward else 1.0)
                                           / (ms_step * 1e-3) / 1e12, 2)
    if with_cpu:
        log("timing the fp64 CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(name, backward=backward, unit=unit)
    return line


PROBE_LIB = os.path.join(ROOT, "attention_fa_fwd_amd", "libfa_probe.so")


def peak_check(iters=100000):
    """The peak re-derived on this device and checked by measurement: compute units and peak
    engine clock from hipDeviceProp (x 4096 dense bf16 FLOP/clk/CU), and a loop of nothing but
    bf16 MFMAs on every SIMD (libfa_probe.so) with the shader clock it ran at."""
    import ctypes

    if not os.path.exists(PROBE_LIB):
        return {"error": "libfa_probe.so not built"}
    lib = ctypes.CDLL(PROBE_LIB)
    lib.fa_probe_device.argtypes = [ctypes.POINTER(ctypes.c_int)] * 2
    lib.fa_probe_mfma.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    rc = lib.fa_probe_device(ctypes.byref(cus), ctypes.byref(khz))
    if rc != 0:
        return {"error": f"fa_probe_device: hip error {rc}"}
    tf, ghz = ctypes.c_double(0.0), ctypes.c_double(0.0)
    rc = lib.fa_probe_mfma(iters, ctypes.byref(tf), ctypes.byref(ghz))
    if rc != 0:
        return {"error": f"fa_probe_mfma: hip error {rc}"}
    derived = cus.value * khz.value * 1e3 * 4096 / 1e12
    return {"cus": cus.value, "max_clock_mhz": round(khz.value / 1e3, 1),
            "derived_peak_tflops": round(derived, 1),
            "mfma_loop_tflops": round(tf.value, 1), "mfma_loop_clock_ghz": round(ghz.value, 3),
            "mfma_loop_frac_of_derived_peak": round(tf.value / derived, 4) if derived else None}


COPY_BYTES = 1 << 30


def calibrate_copy(reps=3):
    """A plain device-to-device copy of COPY_BYTES (torch's copy kernel), for scaling the
    rocprofv3 FETCH_SIZE / WRITE_SIZE counters: the kernel reads and writes COPY_BYTES."""
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {COPY_BYTES} bytes x {reps}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--config", type=int, default=-1, help="force a kernel configuration id")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splitkv", action="store_true",
                    help="time fa_fwd_splitkv with the library's split count")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass fa_bwd (forward results precomputed)")
    ap.add_argument("--cold", action="store_true",
                    help="write 512 MiB between launches (cold L2 and last-level cache) and time "
                         "each launch alone")
    ap.add_argument("--sweep", action="store_true",
                    help="also time causal MHA at B=4, H=32, D=128, fp16, S = 1K..16K (context; "
                         "extra JSON lines on stderr)")
    ap.add_argument("--all", action="store_true",
                    help="also time every named workload (extra JSON lines on stderr)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    a = ap.parse_args(argv)
    if a.calibrate_copy:
        calibrate_copy()
        return 0
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {a.gpus} is not supported "
              "(the attention forward pass here has no multi-GPU path)", file=sys.stderr)
        return 2
    if a.steps < 1 or a.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    from attention_fa_fwd_amd import build as fa_build

    if not os.path.exists(fa_build.LIB_PATH):   # nothing built yet: build it first
        fa_build.build_library(verbose=False)
    if not os.path.exists(fa_build.PROBE_PATH):
        fa_build.build_probe(verbose=False)
    line = bench_line(a.workload, a.steps, a.warmup, a.config, with_cpu=not a.no_cpu_baseline,
                      splitkv=a.splitkv, backward=a.backward, cold=a.cold)
    if line["unit"] == "TFLOP/s":
        log("MFMA peak probe ...")
        line["peak_check"] = peak_check()
    if a.all:
        from attention_fa_fwd_amd.inputs import FP8_WORKLOADS, WORKLOADS

        for name in list(WORKLOADS) + list(FP8_WORKLOADS):
            shape = WORKLOADS.get(name) or FP8_WORKLOADS[name]
            runs = [False, True] if shape["Sq"] <= 16 or shape.get("splitkv_line") else [False]
            for split in runs:
                if name == a.workload and split == a.splitkv:
                    continue
                extra = bench_line(name, a.steps, a.warmup, -1, with_cpu=not a.no_cpu_baseline,
                                   splitkv=split)
                print("[bench-extra] " + json.dumps(extra), file=sys.stderr, flush=True)
        for name in (HEADLINE, "mha_causal_s4096_d128_fp16"):
            extra = bench_line(name, max(1, a.steps // 4), a.warmup, -1,
                               with_cpu=not a.no_cpu_baseline, backward=True)
            print("[bench-extra] " + json.dumps(extra), file=sys.stderr, flush=True)
    if a.sweep:
        from attention_fa_fwd_amd.inputs import SWEEP_WORKLOADS

        for name in SWEEP_WORKLOADS:
            extra = bench_line(name, max(1, a.steps // 4), a.warmup, -1, with_cpu=False)
            print("[bench-extra] " + json.dumps(extra), file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
