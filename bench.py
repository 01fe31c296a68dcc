#!/usr/bin/env python3
"""Benchmark of the SQA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one whole SQA forward (query/key/value projection, attention core,
output projection) through the C ABI (sqa_forward), on synthetic inputs
already resident in HBM. The headline workload is standard SQA at 131072
tokens, causal (H=16, H_q=8, H_kv=4, d_head=64, bf16). This is the middle of the
32k-200k range that the SQA paper's abstract benchmarks. The other long
workloads and their equally shaped MHA/GQA/MQA baselines are timed as well and
reported under "variants", with a sweep of H_kv at fixed H_q (attention time
should not depend on H_kv), a padded batch of sequences of mixed length
(sqa_forward_varlen) and one decode step per sequence over 32k-token key/value
caches (sqa_decode_step; `--decode-only` times just that step), and the
backward pass of the headline workload (sqa_backward; `--backward-only`).

Prints ONE JSON line. FLOPs use the closed form: attention core
4*B*H_q*N^2*d_head (halved when causal) plus the projections
2*B*N*d_model*d_head*(2*H_q + 2*H_kv).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X published dense bf16 MFMA peak
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X published fp32 matrix peak
HBM_PEAK_GBS = 8000.0
HEADLINE = wl.SQA_131K_CAUSAL.name
ATTN_SRC = os.path.join(ROOT, "sparse_query_attention_amd", "csrc", "sqa_attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_hbm_traffic_{}.txt")


def core_flops(w: wl.Workload) -> float:
    f = 4.0 * w.B * w.H_q * float(w.N) ** 2 * w.d_head
    return f / 2 if w.causal else f


def proj_flops(w: wl.Workload) -> float:
    return 2.0 * w.B * w.N * w.d_model * w.d_head * (2 * w.H_q + 2 * w.H_kv)


def attention_bytes(w: wl.Workload) -> int:
    """Algorithmic HBM bytes of one attention launch: read Q, K, V once, write A once."""
    es = 2 if w.dtype == "bf16" else 4
    return es * w.B * w.N * w.d_head * (2 * w.H_q + 2 * w.H_kv)


def proj_bytes(w: wl.Workload):
    """Algorithmic HBM bytes of the two projection launches: (read X and the
    three weights, write Q/K/V) and (read A and Wo, write Y)."""
    es = 2 if w.dtype == "bf16" else 4
    M, D, d = w.B * w.N, w.d_model, w.d_head
    qkv = es * (M * D + D * d * (w.H_q + 2 * w.H_kv) + M * d * (w.H_q + 2 * w.H_kv))
    out = es * (M * w.H_q * d + w.H_q * d * D + M * D)
    return qkv, out


def kernel_source_hash() -> str:
    return hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic(w: wl.Workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = TRAFFIC_FILE.format(w.name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events recorded on the stream the library launches on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e


def run_workload(w: wl.Workload, steps: int, warmup: int, torch, sqa, dev, stage_timing: bool):
    host = wl.to_device_dtype(wl.draw(w), w.dtype)
    d = {k: v.to(dev) for k, v in host.items()}
    del host
    out = torch.empty_like(d["X"])
    stream = torch.cuda.current_stream(dev)
    tm = Timer(torch, stream)

    def step():
        sqa.forward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q, H_kv=w.H_kv,
                    causal=w.causal, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = tm.event()
    for _ in range(steps):
        step()
    e1 = tm.event()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = e0.elapsed_time(e1) / steps
    res = {"ms_per_step": ms, "wall_ms_per_step": wall_ms}

    if stage_timing:
        # The same three kernels through the per-step entry points, with events
        # between them on the launch stream: per-kernel average durations.
        q, k, vt = sqa.qkv_projection(d["X"], d["Wq"], d["Wk"], d["Wv"], H=w.H, H_q=w.H_q,
                                      H_kv=w.H_kv)
        a = sqa.attention(q, k, vt, N=w.N, causal=w.causal)
        y = sqa.output_projection(a, d["Wo"])
        torch.cuda.synchronize()
        tot = {"qkv_projection": 0.0, "attention": 0.0, "output_projection": 0.0}
        for _ in range(steps):
            ev = [tm.event()]
            sqa.qkv_projection(d["X"], d["Wq"], d["Wk"], d["Wv"], H=w.H, H_q=w.H_q, H_kv=w.H_kv,
                               q=q, k=k, vt=vt)
            ev.append(tm.event())
            sqa.attention(q, k, vt, N=w.N, causal=w.causal, a=a)
            ev.append(tm.event())
            sqa.output_projection(a, d["Wo"], out=y)
            ev.append(tm.event())
            torch.cuda.synchronize()
            for i, name in enumerate(tot):
                tot[name] += ev[i].elapsed_time(ev[i + 1])
        res["kernel_ms"] = {k: v / steps for k, v in tot.items()}
        del q, k, vt, a, y
    del d, out
    torch.cuda.empty_cache()
    return res


def run_varlen(w: wl.Workload, steps: int, warmup: int, torch, sqa, dev):
    """sqa_forward_varlen on a padded batch with w's length mix, against
    sqa_forward on the same padded batch (every row treated as a token), timed
    with events on the stream. Rates count the work each call does for real
    tokens: the tokens of each sequence and the causal (or full) query-key
    pairs within it."""
    host = wl.to_device_dtype(wl.draw(w), w.dtype)
    d = {k: v.to(dev) for k, v in host.items()}
    del host
    lens = wl.draw_lens(w)
    stream = torch.cuda.current_stream(dev)
    tm = Timer(torch, stream)
    out = torch.empty_like(d["X"])
    res = {}
    for label, ln in (("varlen", lens), ("padded_dense", np.full(w.B, w.N, dtype=np.int32))):
        lt = torch.from_numpy(ln).to(dev)

        def step():
            if label == "varlen":
                sqa.forward_varlen(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], lt, H=w.H,
                                   H_q=w.H_q, H_kv=w.H_kv, causal=w.causal, out=out)
            else:
                sqa.forward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q,
                            H_kv=w.H_kv, causal=w.causal, out=out)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0 = tm.event()
        for _ in range(steps):
            step()
        e1 = tm.event()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        L = ln.astype(np.float64)
        pairs = float((L * (L + 1) / 2).sum() if w.causal else (L * L).sum())
        core = 4.0 * w.H_q * w.d_head * pairs
        proj = 2.0 * float(L.sum()) * w.d_model * w.d_head * (2 * w.H_q + 2 * w.H_kv)
        res[label] = {"ms_per_step": round(ms, 4),
                      "valid_tokens": int(L.sum()),
                      "tokens_per_s": round(float(L.sum()) / (ms / 1e3), 1),
                      "tflops_valid_work": round((core + proj) / (ms / 1e3) / 1e12, 2)}
    res["lens"] = lens.tolist()
    res["time_vs_padded_dense"] = round(res["varlen"]["ms_per_step"] /
                                        res["padded_dense"]["ms_per_step"], 3)
    del d, out
    torch.cuda.empty_cache()
    return res


# One decode step over 32k-token caches, SQA and its GQA baseline: the step is
# bound by reading the key/value caches, which SQA leaves at H_kv heads, so
# cutting query heads should not speed it up much (abstract).
_DEC = wl.Workload("sqa_bf16_decode_b8_cache32768", B=8, N=32768, d_model=1024, H=16, H_q=8, H_kv=4,
                   causal=True, dtype="bf16", seed=1006)
DECODE_WORKLOADS = (_DEC, _DEC.with_(name=_DEC.name + "_baseline", H_q=16))


def run_decode(w: wl.Workload, steps: int, warmup: int, torch, sqa, dev):
    """sqa_decode_step for B sequences whose caches hold w.N - 1 tokens (filled
    by sqa_prefill): each step attends over w.N keys. Decode reads every cached
    key and value once per step, so its roofline is HBM bandwidth; the bytes
    counted are the caches' rows 0..N-1, the four weight matrices and the
    tokens in and out."""
    host = wl.to_device_dtype(wl.draw(w), w.dtype)
    d = {k: v.to(dev) for k, v in host.items()}
    del host
    es = 2 if w.dtype == "bf16" else 4
    tdt = d["X"].dtype
    kc = torch.empty((w.B, w.H_kv, w.N, w.d_head), dtype=tdt, device=dev)
    vc = torch.empty_like(kc)
    sqa.prefill(d["X"][:, :w.N - 1].contiguous(), d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc, H=w.H,
                H_q=w.H_q, H_kv=w.H_kv)
    x_new = d["X"][:, w.N - 1].contiguous()
    pos = torch.full((w.B,), w.N - 1, dtype=torch.int32, device=dev)
    out = torch.empty_like(x_new)
    del d["X"]
    stream = torch.cuda.current_stream(dev)
    tm = Timer(torch, stream)

    def step():
        sqa.decode_step(x_new, d["Wq"], d["Wk"], d["Wv"], d["Wo"], kc, vc, pos, H=w.H, H_q=w.H_q,
                        H_kv=w.H_kv, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = tm.event()
    for _ in range(steps):
        step()
    e1 = tm.event()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kernel_us = decode_kernel_us(torch, step, steps)
    if kernel_us is not None and not 0.5 * ms * 1e3 <= kernel_us <= ms * 1e3 * 1.02:
        kernel_us = None   # not a sum of this step's kernels (another profiler attached)
    cache_bytes = 2 * w.B * w.H_kv * w.N * w.d_head * es
    weight_bytes = (w.d_model * (w.H_q + 2 * w.H_kv) * w.d_head + w.H_q * w.d_head * w.d_model) * es
    io_bytes = 2 * w.B * w.d_model * es
    total = cache_bytes + weight_bytes + io_bytes
    del d, kc, vc
    torch.cuda.empty_cache()
    return {"B": w.B, "cache_tokens": w.N, "H_q": w.H_q, "H_kv": w.H_kv,
            "ms_per_step": round(ms, 4), "tokens_per_s": round(w.B / (ms / 1e3), 1),
            "bytes_per_step": total, "gbs": round(total / (ms / 1e3) / 1e9, 1),
            "frac_hbm_peak": round(total / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_us_per_step": None if kernel_us is None else round(kernel_us, 2),
            "kernel_frac_hbm_peak": None if kernel_us is None else
            round(total / (kernel_us / 1e6) / 1e9 / HBM_PEAK_GBS, 4)}


def decode_kernel_us(torch, step, steps: int):
    """Device time of the decode step's own kernels per step (the sum of their
    durations, without the gaps between launches), from torch's profiler over
    `steps` more steps. The profiler records every HIP kernel of the process,
    the library's included. None unless it saw the same number of kernels in
    every step (3 or 4 launches); under another profiler (rocprofv3) it sees
    only some."""
    try:
        from torch.profiler import ProfilerActivity, profile
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
        kernels = [ev for ev in prof.key_averages() if getattr(ev, "device_time_total", 0.0) > 0]
        total = sum(ev.device_time_total for ev in kernels)
        launches = sum(ev.count for ev in kernels)
    except Exception:   # profiler unavailable: report the step time only
        return None
    if total <= 0 or launches not in (3 * steps, 4 * steps):
        return None
    return total / steps


def run_backward(w: wl.Workload, steps: int, warmup: int, torch, sqa, dev):
    """A training step of the layer on w with a seeded upstream gradient:
    sqa_forward_train, then sqa_backward from its saved activations (also
    timed recomputing them), with events on the launch stream. Algorithmic
    work of the backward: the attention backward's five score-sized products
    (2.5x the forward core) and the projection gradients (dA, dWo, dX and the
    three input-weight gradients: 2x the forward projections)."""
    arrays = wl.draw(w)
    arrays["dY"] = wl.draw_upstream_grad(w)
    host = wl.to_device_dtype(arrays, w.dtype)
    d = {k: v.to(dev) for k, v in host.items()}
    del host, arrays
    outs = (torch.empty_like(d["X"]), torch.empty_like(d["Wq"]), torch.empty_like(d["Wk"]),
            torch.empty_like(d["Wv"]), torch.empty_like(d["Wo"]))
    stream = torch.cuda.current_stream(dev)
    tm = Timer(torch, stream)

    y = torch.empty_like(d["X"])
    _, saved = sqa.forward_train(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q,
                                 H_kv=w.H_kv, causal=w.causal, out=y)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = tm.event()
        for _ in range(steps):
            fn()
        e1 = tm.event()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def fwd_train():
        sqa.forward_train(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], H=w.H, H_q=w.H_q,
                          H_kv=w.H_kv, causal=w.causal, out=y)

    def bwd(sv):
        return lambda: sqa.backward(d["X"], d["Wq"], d["Wk"], d["Wv"], d["Wo"], d["dY"], H=w.H,
                                    H_q=w.H_q, H_kv=w.H_kv, causal=w.causal, saved=sv, out=outs)

    ms = timed(bwd(saved))            # from the training forward's activations
    ms_re = timed(bwd(None))          # recomputing them
    ms_fwd = timed(fwd_train)
    flop = 2.5 * core_flops(w) + 2.0 * proj_flops(w)
    res = {"ms": round(ms, 4), "tflops_algorithmic": round(flop / (ms / 1e3) / 1e12, 2),
           "algorithmic_flop": flop, "ms_recomputing_activations": round(ms_re, 4),
           "forward_train_ms": round(ms_fwd, 4),
           "training_step_ms": round(ms_fwd + ms, 4),
           "training_tokens_per_s": round(w.tokens / ((ms_fwd + ms) / 1e3), 1)}
    del d, outs, saved, y
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    """The host CPU's model name (the first "model name" of /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: wl.Workload, rows_sample: int = 24576):
    """The float64 oracle on a bounded sample: every key/value projection of the
    workload, plus the whole forward of `rows_sample` evenly spaced query rows.
    The time is extrapolated linearly to all B*N rows."""
    import numpy as np
    import oracle
    host = wl.to_device_dtype(wl.draw(w), w.dtype)
    o = {k: wl.widen(v) for k, v in host.items()}
    del host
    cores = len(os.sched_getaffinity(0))
    rows = ((np.arange(rows_sample) + 0.5) * (w.B * w.N) / rows_sample).astype(np.int64)
    cache = {}
    t0 = time.perf_counter()
    oracle.sqa_forward_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv, w.d_head,
                            w.causal, bf16=(w.dtype == "bf16"), rows=rows[:1], kv_cache=cache,
                            workers=cores)
    t_kv = time.perf_counter() - t0          # key/value projection of every token (+ one row)
    t1 = time.perf_counter()
    oracle.sqa_forward_rows(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv, w.d_head,
                            w.causal, bf16=(w.dtype == "bf16"), rows=rows, kv_cache=cache,
                            workers=cores)
    t_rows = time.perf_counter() - t1
    full_s = t_kv + t_rows * (w.B * w.N) / rows_sample
    return {"value": (w.B * w.N) / full_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"float64 oracle: key/value projection of all {w.B * w.N} tokens "
                       f"({t_kv:.1f} s) + full forward of {rows_sample} evenly spaced query rows "
                       f"({t_rows:.1f} s), extrapolated linearly to {w.B * w.N} rows "
                       f"= {full_s:.0f} s per step"),
            "seconds_measured": round(t_kv + t_rows, 2)}


def _oracle_inputs(w: wl.Workload, n: int = None, grad: bool = False):
    """w's seeded inputs rounded to its dtype and widened to float64, the first
    n tokens of each sequence when n is given."""
    arrays = wl.draw(w)
    if grad:
        arrays["dY"] = wl.draw_upstream_grad(w)
    if n is not None:
        for k in ("X", "dY"):
            if k in arrays:
                arrays[k] = arrays[k][:, :n]
    host = wl.to_device_dtype(arrays, w.dtype)
    return {k: wl.widen(v) for k, v in host.items()}


def cpu_baseline_decode(w: wl.Workload):
    """The float64 oracle on one decode step: the forward of the B new tokens'
    rows (position N-1) against all N cached keys and values. The keys and
    values are projected first, untimed, as the cache that prefill fills."""
    import numpy as np
    import oracle
    o = _oracle_inputs(w)
    cores = len(os.sched_getaffinity(0))
    rows = np.arange(w.B, dtype=np.int64) * w.N + (w.N - 1)
    cache = {}
    args = (o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv, w.d_head, w.causal)
    oracle.sqa_forward_rows(*args, bf16=(w.dtype == "bf16"), rows=rows, kv_cache=cache, workers=cores)
    t0 = time.perf_counter()
    oracle.sqa_forward_rows(*args, bf16=(w.dtype == "bf16"), rows=rows, kv_cache=cache, workers=cores)
    t = time.perf_counter() - t0
    return {"value": round(w.B / t, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"float64 oracle: one decode step, {w.B} new rows against {w.N} cached keys "
                       f"each ({t * 1e3:.0f} ms; the cache projection untimed)"),
            "seconds_measured": round(t, 3)}


def cpu_baseline_backward(w: wl.Workload, sizes=(4096, 8192), reps: int = 2):
    """The float64 oracle backward (gradients of x and the four weights) on
    the first n tokens of the workload for two n (the faster of `reps` runs
    each), fitted as a*n + b*n^2 (projections, attention) and extrapolated to
    all N tokens. The sizes are large enough for the quadratic part to show
    above the timing noise."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    ts = []
    for n in sizes:
        o = _oracle_inputs(w, n, grad=True)
        best = float("inf")
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.sqa_backward(o["X"], o["Wq"], o["Wk"], o["Wv"], o["Wo"], o["dY"], w.H_q, w.H_kv,
                                w.d_head, w.causal, bf16=(w.dtype == "bf16"), workers=cores)
            best = min(best, time.perf_counter() - t0)
        ts.append(best)
    (n1, n2), (t1, t2) = sizes, ts
    b = max(0.0, (t2 / n2 - t1 / n1) / (n2 - n1))
    a = max(0.0, t1 / n1 - b * n1)
    full = a * w.N + b * w.N * w.N
    return {"value": round(w.tokens / full, 2), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": (f"float64 oracle backward on the first {n1} and {n2} tokens ({t1:.1f} s, "
                       f"{t2:.1f} s), fitted as a*n + b*n^2 and extrapolated to {w.N} tokens "
                       f"= {full:.0f} s per step"),
            "seconds_measured": round(reps * (t1 + t2), 2)}


def cpu_baseline_varlen(w: wl.Workload, rows_per_seq: int = 1024):
    """The float64 oracle on each sequence of w's length mix: its key/value
    projection plus the forward of rows_per_seq evenly spaced rows, the row
    time extrapolated linearly to the sequence's length."""
    import numpy as np
    import oracle
    o = _oracle_inputs(w)
    lens = wl.draw_lens(w)
    cores = len(os.sched_getaffinity(0))
    measured = full = 0.0
    for b, L in enumerate(int(x) for x in lens):
        if L == 0:
            continue
        k = min(rows_per_seq, L)
        rows = ((np.arange(k) + 0.5) * L / k).astype(np.int64)
        args = (o["X"][b:b + 1, :L], o["Wq"], o["Wk"], o["Wv"], o["Wo"], w.H_q, w.H_kv, w.d_head,
                w.causal)
        cache = {}
        t0 = time.perf_counter()
        oracle.sqa_forward_rows(*args, bf16=(w.dtype == "bf16"), rows=rows[:1], kv_cache=cache,
                                workers=cores)
        t_kv = time.perf_counter() - t0
        t1 = time.perf_counter()
        oracle.sqa_forward_rows(*args, bf16=(w.dtype == "bf16"), rows=rows, kv_cache=cache,
                                workers=cores)
        t_rows = time.perf_counter() - t1
        measured += t_kv + t_rows
        full += t_kv + t_rows * L / k
    total = int(lens.sum())
    return {"value": round(total / full, 1), "unit": "valid tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": (f"float64 oracle: per sequence, the key/value projection plus {rows_per_seq} "
                       f"evenly spaced rows, extrapolated to its length; {total} valid tokens "
                       f"= {full:.0f} s per step"),
            "seconds_measured": round(measured, 2)}


def calibrate_copy(torch, dev, nbytes: int = 1 << 30, reps: int = 3):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE and
    WRITE_SIZE readings to bytes."""
    x = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(wl.WORKLOADS))
    ap.add_argument("--no-variants", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=24576)
    ap.add_argument("--backward-only", action="store_true",
                    help="only time sqa_backward on the workload")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time the decode step (B=8, 32k-token caches), SQA and GQA baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (rocprofv3 counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this SQA forward path has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_query_attention_amd as sqa
    sqa._lib.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(torch, dev)
        return
    if args.backward_only:
        w = wl.WORKLOADS[args.workload]
        print(json.dumps({w.name + "_backward": run_backward(w, args.steps, args.warmup, torch, sqa,
                                                              dev)}), flush=True)
        return
    if args.decode_only:
        for v in DECODE_WORKLOADS:
            print(json.dumps({v.name: run_decode(v, args.steps, args.warmup, torch, sqa, dev)}),
                  flush=True)
        return

    w = wl.WORKLOADS[args.workload]
    main_res = run_workload(w, args.steps, args.warmup, torch, sqa, dev, stage_timing=True)
    ms = main_res["ms_per_step"]
    tokens_s = w.tokens / (ms / 1e3)
    cf, pf = core_flops(w), proj_flops(w)
    attn_ms = main_res["kernel_ms"]["attention"]
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    achieved = cf / (attn_ms / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(w),
                "kernel": "attn_kernel (attention core)",
                "algorithmic_flop_per_launch": cf, "algorithmic_bytes_per_launch": attention_bytes(w),
                "avg_launch_ms": round(attn_ms, 4)}

    variants = {}
    if not args.no_variants:
        vsteps, vwarm = max(3, args.steps // 2), max(1, args.warmup)
        # The short 16 x 1024 training-shaped workload runs in tens of
        # microseconds: more steps keep its timed region near 10 ms.
        short = (wl.SSQA_1K_CAUSAL.name, wl.SSQA_1K_CAUSAL.baseline().name)
        for v in (wl.SSQA_1K_CAUSAL, wl.SSQA_1K_CAUSAL.baseline(),
                  wl.XSQA_32K, wl.XSQA_32K.baseline(), wl.SQA_131K_CAUSAL.baseline(),
                  wl.XSMQA_200K, wl.XSMQA_200K.baseline()):
            if v.name == w.name:
                continue
            n_steps = max(200, vsteps) if v.name in short else vsteps
            r = run_workload(v, n_steps, max(10, vwarm) if v.name in short else vwarm, torch, sqa,
                             dev, stage_timing=True)
            am = r["kernel_ms"]["attention"]
            variants[v.name] = {
                "H_q": v.H_q, "H_kv": v.H_kv, "N": v.N, "causal": v.causal,
                "ms_per_step": round(r["ms_per_step"], 4),
                "tokens_per_s": round(v.tokens / (r["ms_per_step"] / 1e3), 1),
                "attention_ms": round(am, 4),
                "attention_tflops": round(core_flops(v) / (am / 1e3) / 1e12, 2),
                "total_tflops": round((core_flops(v) + proj_flops(v)) / (r["ms_per_step"] / 1e3) / 1e12, 2)}
        for v in (wl.SSQA_1K_CAUSAL, wl.XSQA_32K, wl.SQA_131K_CAUSAL, wl.XSMQA_200K):
            b = v.baseline()
            sv = variants.get(v.name) or ({"attention_ms": attn_ms, "ms_per_step": ms}
                                          if v.name == w.name else None)
            sb = variants.get(b.name)
            if sv and sb:
                key = v.name + "_speedup_vs_baseline"
                variants[key] = {"attention": round(sb["attention_ms"] / sv["attention_ms"], 3),
                                 "whole_forward": round(sb["ms_per_step"] / sv["ms_per_step"], 3),
                                 "ideal_H_over_H_q": b.H_q / v.H_q}
        # Attention time at fixed H_q = 4 as H_kv shrinks 4 -> 2 -> 1. Score FLOPs
        # depend on H_q alone, so fewer key/value heads should not cut the core
        # time (ReactiveAI/xSMQAT-m model card, description and conclusion: xSMQA
        # trains no faster than xSQA).
        sweep = {}
        for hkv in (4, 2, 1):
            v = wl.XSQA_32K.with_(name=f"xsqa_bf16_n32768_hkv{hkv}", H_kv=hkv,
                                  baseline_H_q=None, baseline_H_kv=None)
            r = run_workload(v, vsteps, vwarm, torch, sqa, dev, stage_timing=True)
            sweep[f"H_kv={hkv}"] = round(r["kernel_ms"]["attention"], 4)
        times = list(sweep.values())
        variants["hkv_sweep_n32768_hq4_attention_ms"] = dict(
            sweep, max_over_min=round(max(times) / min(times), 3))
        for v in DECODE_WORKLOADS:
            variants[v.name] = run_decode(v, max(10, args.steps), vwarm, torch, sqa, dev)
        # Training: the gradients of the headline workload (sqa_backward), and
        # forward + backward as one training step of the layer.
        variants[w.name + "_backward"] = run_backward(w, vsteps, vwarm, torch, sqa, dev)
        # A padded batch of sequences of mixed length (sqa_forward_varlen).
        variants[wl.SQA_VARLEN_32K.name] = run_varlen(wl.SQA_VARLEN_32K, vsteps, vwarm, torch, sqa,
                                                      dev)

    line = {
        "metric": "SQA fwd tokens/s + TFLOP/s (% bf16 MFMA peak) at N=32k-200k, 1 GPU",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/d_model) weights)",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "d_model": w.d_model, "H": w.H,
                   "H_q": w.H_q, "H_kv": w.H_kv, "d_head": w.d_head, "causal": w.causal,
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "single GPU"},
        "tflops_total": round((cf + pf) / (ms / 1e3) / 1e12, 2),
        "tflops_attention": round(achieved, 2),
        "pct_bf16_peak_attention": round(100 * achieved / peak, 2),
        "kernel_ms": {k: round(v, 4) for k, v in main_res["kernel_ms"].items()},
        "projection_gbs": {
            "qkv_projection": round(proj_bytes(w)[0] / (main_res["kernel_ms"]["qkv_projection"] / 1e3) / 1e9, 1),
            "output_projection": round(proj_bytes(w)[1] / (main_res["kernel_ms"]["output_projection"] / 1e3) / 1e9, 1)},
        "roofline": roofline,
        "variants": variants,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
        # the same oracle beside the other rows of the path, on bounded samples
        if not args.no_variants:
            variants[DECODE_WORKLOADS[0].name]["cpu_baseline"] = cpu_baseline_decode(DECODE_WORKLOADS[0])
            variants[w.name + "_backward"]["cpu_baseline"] = cpu_baseline_backward(w)
            variants[wl.SQA_VARLEN_32K.name]["cpu_baseline"] = cpu_baseline_varlen(wl.SQA_VARLEN_32K)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
