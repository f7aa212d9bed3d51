#!/usr/bin/env python3
"""Benchmark of the fused mixed-head SAF attention layer on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input held in HBM: the
mixed forward (ordinary and replaced heads in one grid) followed by the mixed backward (delta
preprocess, key-block kernel, query-block dQ kernel; bf16 at d=128 with the workspace that keeps dS
between the two, the key-block kernel also stores dS and the dQ kernel reads it).  Forward-only workloads (prefill) time the
forward alone.  Prints ONE JSON line.

The headline workload is the largest fwd+bwd configuration that fits one GPU: one GPU's share of
the pages' 1B-model run, B=2, H=16 heads of width 128, T=8192, bf16, 4 of 16 heads replaced
([Notes §四.6]; [Paper page] Table 23).  The same line carries, under "configs", the other layer
shapes the pages time: the 124M-shaped layer at 4K (B=8, 3 of 12 heads replaced) and 8K (B=4, 6 of
12 replaced), fwd+bwd ([Paper page] Table 2), and causal prefill at B=64, T=4096 and B=2, T=16384,
forward only ([Paper page] Table 29), each also with all heads ordinary and all replaced.
Algorithmic flops per (batch, head) over the T(T+1)/2 causal entries: ordinary forward 4d,
ordinary backward 10d, replaced forward 2d, replaced backward 2d per entry.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-variants]
                  [--no-configs]

[Notes] = "When Can Attention Heads Be Statically Defined?：中文精读笔记";
[Paper page] = "When Can Attention Heads Be Statically Defined?".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "mixed-head attn fwd+bwd tokens/s and TFLOP/s at 1 GPU; % of bf16 MFMA peak"
# MI355X dense bf16 matrix peak: 256 CUs x 2.4 GHz x 4096 flop/clk/CU (AMD's published 2.5 PFLOP/s)
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


def kernel_flops(B, T, d, replaced):
    """Algorithmic flops of one launch of each kernel (GEMM work the method defines)."""
    c = T * (T + 1) / 2.0
    n_rep = sum(1 for x in replaced if x)
    n_ord = len(replaced) - n_rep
    return {
        "mixed_fwd": B * c * (n_ord * 4 * d + n_rep * 2 * d),    # S, PV (ordinary); PV (replaced)
        "bwd_kv": B * c * (n_ord * 8 * d + n_rep * 2 * d),      # S, dP, dV, dK; dV (replaced)
        "bwd_dq": B * c * (n_ord * 2 * d),                   # dQ (S, dP re-formed: not counted)
        "bwd_dq_ds": B * c * (n_ord * 2 * d),                # dQ from the stored dS
        "bwd_pre": 0.0,
    }


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter record
    (profiles/hbm_traffic.json), or None if there is none or the kernel's source files changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload, {}).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for fn in rec["sources"]:
        with open(os.path.join(ROOT, "fixed_pattern_mixed_amd", "csrc", fn), "rb") as f:
            h.update(f.read())
    return rec["bytes"] if h.hexdigest() == rec["source_sha256"] else None


def total_flops(B, T, d, replaced, backward):
    kf = kernel_flops(B, T, d, replaced)
    return kf["mixed_fwd"] + (kf["bwd_kv"] + kf["bwd_dq"] if backward else 0.0)  # one dQ kernel runs


class Layer:
    """Preallocated buffers and raw C-ABI calls for one layer shape (no allocation per step).
    draw_on="cuda" draws the synthetic inputs on the GPU (same distributions, no host work)."""

    def __init__(self, saf, torch, w, replaced, dev, draw_on=None):
        import synth
        self.saf, self.w, self.rep = saf, w, list(replaced)
        x = synth.layer_inputs(w.B, w.H, w.T, w.d, w.torch_dtype, replaced, w.ar_std,
                               synth.SEED0 + w.index, backward=True, device=dev, Hkv=w.Hkv or None,
                               draw_on=draw_on)
        self.x = x
        B, H, T, d = w.B, w.H, w.T, w.d
        self.Hkv = w.kv_heads
        self.o = torch.empty_like(x.q)
        self.lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
        self.dq = torch.empty_like(x.q)
        self.dk, self.dv = torch.empty_like(x.k), torch.empty_like(x.v)
        self.dt = saf.SAF_BF16 if w.dtype == "bf16" else saf.SAF_F32
        # the backward workspace with room for the stored dS where the library keeps it (bf16,
        # d = 128, no grouped heads); nb_min: the smaller one, with which dQ re-forms S and dP
        self.nb_min = max(saf.saf_attn_bwd_workspace_size(B, H, T, d), 256)
        nb = saf.saf_attn_bwd_ds_workspace_size(self.dt, B, H, self.Hkv, T, d, sum(1 for x in replaced if x))
        nb = nb if self.nb_min < nb <= self.nb_min + saf.DS_WORKSPACE_MAX else self.nb_min
        nf = max(saf.saf_attn_fwd_workspace_size(B, H, T, d), 256)
        self.ws_b = torch.empty(nb, dtype=torch.uint8, device=dev)
        self.ws_f = torch.empty(nf, dtype=torch.uint8, device=dev)
        self.nb, self.nf = nb, nf
        self.recompute_ds = False  # True: pass the smaller workspace (dQ re-forms S and dP)
        self.mask = saf._mask(replaced, H)
        self.stream = torch.cuda.current_stream(dev).cuda_stream
        # the replaced heads' pattern is a frozen buffer: its normaliser is prepared once, as when
        # the pattern is installed, and reused by every step
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.pattern = saf.prepare_pattern(replaced, x.a, x.r)
        torch.cuda.synchronize()
        self.prepare_ms = (time.perf_counter() - t0) * 1e3

    def fwd(self, stream=None):
        s, w, x = self.saf, self.w, self.x
        st = s.saf_attn_fwd_gqa(self.dt, w.B, w.H, self.Hkv, w.T, w.d, x.q.data_ptr(),
                                x.k.data_ptr(), x.v.data_ptr(), self.mask, x.a.data_ptr(),
                                x.r.data_ptr(), x.a.shape[1], self.pattern.data_ptr(), 0.0,
                                self.o.data_ptr(), self.lse.data_ptr(), self.ws_f.data_ptr(),
                                self.nf, self.stream if stream is None else stream)
        s._check(st, "saf_attn_fwd")

    def bwd(self):
        s, w, x = self.saf, self.w, self.x
        nb = self.nb_min if self.recompute_ds else self.nb
        st = s.saf_attn_bwd_gqa(self.dt, w.B, w.H, self.Hkv, w.T, w.d, x.q.data_ptr(),
                                x.k.data_ptr(), x.v.data_ptr(), self.o.data_ptr(),
                                x.dout.data_ptr(), self.lse.data_ptr(), self.mask, x.a.data_ptr(),
                                x.r.data_ptr(), x.a.shape[1], self.pattern.data_ptr(), 0.0,
                                self.dq.data_ptr(), self.dk.data_ptr(), self.dv.data_ptr(),
                                self.ws_b.data_ptr(), nb, self.stream)
        s._check(st, "saf_attn_bwd")

    def step(self):
        self.fwd()
        if self.w.backward:
            self.bwd()


def spin_up(torch, seconds=0.3):
    """Bring the GPU out of its idle clocks before anything is timed: a plain bf16 matrix product
    loop for `seconds` (not part of the hot path; the W warm-up steps and K timed steps follow).
    Without it the first few milliseconds of timing run at ramping clocks.  Returns the loop's
    duration (ms) and the library GEMM's rate over its last 8 products (TFLOP/s): a reference for
    what the matrix cores sustain on this board with a vendor-tuned dense product."""
    a = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
    t0 = time.perf_counter()
    n = 0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while time.perf_counter() - t0 < seconds:
        ev0.record()
        for _ in range(8):
            b = a @ a
        ev1.record()
        torch.cuda.synchronize()
        n += 8
    gemm = 8 * 2.0 * 8192 ** 3 / (ev0.elapsed_time(ev1) * 1e-3) / 1e12
    del a, b
    return round((time.perf_counter() - t0) * 1e3, 1), round(gemm, 1)


def time_steps(torch, layer, steps, warmup, trace=None, per_step=None):
    """Seconds per step over `steps` steps after `warmup` untimed ones.  per_step: a list that
    receives each step's duration in ms, from HIP events recorded between the steps on the stream
    the library launches on."""
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    if trace is not None:
        trace.begin()
    ev = None
    if per_step is not None:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
    t0 = time.perf_counter()
    for i in range(steps):
        layer.step()
        if ev is not None:
            ev[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if trace is not None:
        trace.end()
        trace.collect()
    if ev is not None:
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return (t1 - t0) / steps


def calibration(torch, saf, w, steps=3):
    """Time saf_calibrate on the workload's calibration shape (N sequences of its H, T, d; Q, K
    N(0,1) bf16, drawn on the GPU).  Algorithmic work: two passes of s Q K^T over the causal entries
    (row statistics, then the mean / deviation tiles): 4d flops per entry per sequence per head."""
    N, H, T, d = w.calib_N, w.H, w.T, w.d
    g = torch.Generator(device="cuda").manual_seed(1437)
    q = torch.randn((N, H, T, d), device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((N, H, T, d), device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
    ahat = torch.empty((H, T, T), dtype=torch.float32, device="cuda")
    svar = torch.empty((H,), dtype=torch.float64, device="cuda")
    nws = saf.saf_calibrate_workspace_size(N, H, T, d)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    call = lambda: saf._check(saf.saf_calibrate(saf.SAF_BF16, N, H, T, d, q.data_ptr(), k.data_ptr(),  # noqa: E731
                                                0.0, ahat.data_ptr(), svar.data_ptr(), None, ws.data_ptr(),
                                                nws, stream), "saf_calibrate")
    call()
    torch.cuda.synchronize()
    trace = saf.KernelTrace(capacity=4 * steps)
    trace.begin()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    trace.end()
    trace.collect()
    c = T * (T + 1) / 2.0
    kf = {"calib_lse": N * H * c * 2 * d, "calib_stats": N * H * c * 2 * d, "calib_reduce": 0.0}
    kernels = {}
    for name, st in trace.summary().items():
        ent = {"avg_ms": round(st["avg_ms"], 4), "launches": st["launches"]}
        if kf.get(name):
            ent["tflops"] = round(kf[name] / (st["avg_ms"] * 1e-3) / 1e12, 1)
        kernels[name] = ent
    dom = max(trace.summary().items(), key=lambda kv: kv[1]["total_ms"])[0]
    ach = kf[dom] / (trace.summary()[dom]["avg_ms"] * 1e-3) / 1e12
    trace.close()
    flops = kf["calib_lse"] + kf["calib_stats"]
    fit = fit_timing(torch, saf, ahat, stream)
    return {"workload": "%s calibration: N=%d, H=%d, T=%d, d=%d, bf16" % (w.name, N, H, T, d),
            "fit": fit,
            "ms": round(dt * 1e3, 3), "tflops": round(flops / dt / 1e12, 1),
            "pct_bf16_peak": round(100 * flops / dt / 1e12 / PEAK_BF16_TFLOPS, 2),
            "ahat_write_gbs": round(4.0 * H * T * T / dt / 1e9, 1), "kernels": kernels,
            "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic(w.name + "_calibration", dom)}}


def pattern_gradient(torch, saf, layer, steps):
    """Time saf_attn_bwd_pattern (dL/da, dL/dr of the replaced heads, for a pattern that is trained
    instead of frozen: [Paper page] Table 14) on the layer's own forward outputs.  Algorithmic
    work: G = dO V^T over the replaced heads' causal entries, 2d flops per entry."""
    w, x = layer.w, layer.x
    B, H, T, d = w.B, w.H, w.T, w.d
    n_rep = sum(1 for z in layer.rep if z)
    if n_rep == 0 or not w.backward:
        return None
    layer.fwd()
    da, dr = torch.zeros_like(x.a), torch.zeros_like(x.r)
    nws = saf.saf_attn_bwd_pattern_workspace_size(B, H, T, d)
    ws = torch.empty(nws, dtype=torch.uint8, device=x.v.device)
    call = lambda: saf._check(saf.saf_attn_bwd_pattern(  # noqa: E731
        layer.dt, B, H, T, d, x.v.data_ptr(), layer.o.data_ptr(), x.dout.data_ptr(),
        layer.lse.data_ptr(), layer.mask, x.a.data_ptr(), x.r.data_ptr(), x.a.shape[1],
        layer.pattern.data_ptr(), da.data_ptr(), dr.data_ptr(), ws.data_ptr(), nws,
        layer.stream), "saf_attn_bwd_pattern")
    call()
    torch.cuda.synchronize()
    trace = saf.KernelTrace(capacity=4 * steps)
    trace.begin()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    trace.end()
    trace.collect()
    flops = B * n_rep * (T * (T + 1) / 2.0) * 2 * d
    kernels = {}
    for name, st in trace.summary().items():
        ent = {"avg_ms": round(st["avg_ms"], 4), "launches": st["launches"]}
        if name == "bwd_pattern":
            ent["tflops"] = round(flops / (st["avg_ms"] * 1e-3) / 1e12, 1)
        kernels[name] = ent
    trace.close()
    return {"ms": round(dt * 1e3, 4), "kernels": kernels}


def prefill_latency(torch, saf, dev, name="prefill_b1_t4096", reps=50):
    """Small-batch prefill (B=1, T=4096, forward only), where the pages see launch overhead
    dominate ([Notes §四]; Appendix D.3): one forward call timed three ways -- back to back on the
    stream, replayed from a HIP graph that captured it, and one call followed by a synchronize
    (median).  With the pattern prepared the call is a single kernel launch."""
    import synth
    w = synth.WORKLOADS[name]
    lay = Layer(saf, torch, w, w.replaced(), dev)
    for _ in range(5):
        lay.fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        lay.fwd()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / reps
    singles = []
    for _ in range(21):
        t0 = time.perf_counter()
        lay.fwd()
        torch.cuda.synchronize()
        singles.append(time.perf_counter() - t0)
    singles.sort()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        lay.fwd(stream=cs.cuda_stream)  # warm the capture stream
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cs):
        lay.fwd(stream=cs.cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    graph = (time.perf_counter() - t0) / reps
    flops = total_flops(w.B, w.T, w.d, w.replaced(), False)
    return {"workload": "%s: B=%d, H=%d, T=%d, d=%d, bf16, fwd" % (w.name, w.B, w.H, w.T, w.d),
            "eager_ms": round(eager * 1e3, 4), "graph_replay_ms": round(graph * 1e3, 4),
            "call_and_sync_median_ms": round(singles[len(singles) // 2] * 1e3, 4),
            "tokens_per_s_graph": round(w.B * w.T / graph, 1),
            "tflops_graph": round(flops / graph / 1e12, 1)}


def fit_timing(torch, saf, ahat, stream, steps=400, lr=0.1, reps=2):
    """Time saf_fit_pattern (400 Adam steps on the row-wise cross-entropy, fp64) on the
    calibration's mean maps, every head fitted.  Per step: three length-T causal convolutions per
    head (3 T(T+1)/2 fp64 multiply-adds); the marginal pass reads ahat once (4 T^2 bytes per head)."""
    H, T, _ = ahat.shape
    a = torch.empty((H, T), dtype=torch.float32, device=ahat.device)
    r = torch.empty_like(a)
    kl = torch.empty((H,), dtype=torch.float64, device=ahat.device)
    nws = saf.saf_fit_pattern_workspace_size(H, T)
    ws = torch.empty(nws, dtype=torch.uint8, device=ahat.device)
    call = lambda: saf._check(saf.saf_fit_pattern(H, T, ahat.data_ptr(), steps, lr, a.data_ptr(),  # noqa: E731
                                                  r.data_ptr(), kl.data_ptr(), None, ws.data_ptr(),
                                                  nws, stream), "saf_fit_pattern")
    call()
    torch.cuda.synchronize()
    trace = saf.KernelTrace(capacity=(2 * steps + 8) * reps)
    trace.begin()
    t0 = time.perf_counter()
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    trace.end()
    trace.collect()
    kernels = {name: {"avg_ms": round(st["avg_ms"], 4), "launches": st["launches"]}
               for name, st in trace.summary().items()}
    trace.close()
    fma = 3.0 * H * T * (T + 1) / 2.0 * steps
    klh = kl.cpu().tolist()
    return {"heads": H, "T": T, "steps": steps, "lr": lr, "ms": round(dt * 1e3, 3),
            "fp64_tflops": round(2 * fma / dt / 1e12, 2), "kernels": kernels,
            "kl_min": round(min(klh), 4), "kl_max": round(max(klh), 4),
            "accepted_at_0.2_nat": sum(1 for x in klh if x <= 0.2)}


def cpu_model():
    """The host CPU's model name with its family / model / stepping numbers (from /proc/cpuinfo, as
    lscpu reports them: some hosts give only a family name)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ":" not in ln:
                    if info:
                        break  # the first processor's block is enough
                    continue
                k, v = (t.strip() for t in ln.split(":", 1))
                info.setdefault(k, v)
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    ids = ["%s %s" % (k, info[k]) for k in ("cpu family", "model", "stepping") if k in info]
    return "%s (%s)" % (name, ", ".join(ids)) if ids else name


def cpu_baseline(w, replaced, min_seconds=10.0):
    """The fp64 oracle, as it stands, on whole sequences of the same workload (all heads, full T),
    one after another until at least min_seconds of CPU work (or the whole batch) is done."""
    import oracle
    import synth
    x = synth.layer_inputs(w.B, w.H, w.T, w.d, w.torch_dtype, replaced, w.ar_std,
                           synth.SEED0 + w.index, backward=w.backward, Hkv=w.Hkv or None)
    oracle.build()
    n_seq, dt = 0, 0.0
    while n_seq < w.B and dt < min_seconds:
        heads = [(n_seq, h) for h in range(w.H)]
        t0 = time.perf_counter()
        if w.Hkv:
            oracle.layer_fwd_gqa(x.q, x.k, x.v, replaced, x.a, x.r, heads=heads)
            if w.backward:
                oracle.layer_bwd_gqa(x.q, x.k, x.v, x.dout, replaced, x.a, x.r, batches=[n_seq])
        else:
            oracle.layer_fwd(x.q, x.k, x.v, replaced, x.a, x.r, heads=heads)
            if w.backward:
                oracle.layer_bwd(x.q, x.k, x.v, x.dout, replaced, x.a, x.r, heads=heads)
        dt += time.perf_counter() - t0
        n_seq += 1
    return {
        "value": round(n_seq * w.T / dt, 1),
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": "%d of %d sequences (all %d heads, full T=%d, %s) in %.1f s"
                  % (n_seq, w.B, w.H, w.T, "fwd+bwd" if w.backward else "fwd", dt),
    }


def backward_unit(kernels, kf):
    """The backward's kernels as one unit (the preprocess, the key-block kernel and whichever dQ
    kernel ran): summed average durations and their algorithmic flops (dQ counted once)."""
    names = [k for k in ("bwd_pre", "bwd_kv", "bwd_dq", "bwd_dq_ds", "bwd_dv_rep") if k in kernels]
    if "bwd_kv" not in names:
        return None
    ms = sum(kernels[k]["avg_ms"] for k in names)
    fl = kf["bwd_kv"] + kf["bwd_dq"]
    return {"kernels": names, "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
            "pct_bf16_peak": round(100 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}


def step_spread(per_step):
    """Median, minimum and maximum of the per-step durations (ms)."""
    v = sorted(per_step)
    if not v:
        return None
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"median": round(med, 4), "min": round(v[0], 4), "max": round(v[-1], 4), "n": n}


def cpu_calibration_baseline(w, min_seconds=10.0):
    """The fp64 oracle's calibration (Eq. (1) rows and the mean map) on whole heads of the
    workload's calibration shape (all N sequences, full T; Q, K N(0,1) rounded to bf16), one head
    after another until at least min_seconds of CPU work (or every head) is done, scaled to all
    heads: estimated ms per saf_calibrate call of the same shape."""
    import oracle
    import torch
    N, H, T, d = w.calib_N, w.H, w.T, w.d
    g = torch.Generator().manual_seed(1437)
    oracle.build()
    n_h, dt = 0, 0.0
    while n_h < H and dt < min_seconds:
        q = torch.randn((N, T, d), generator=g).to(torch.bfloat16).double().numpy()
        k = torch.randn((N, T, d), generator=g).to(torch.bfloat16).double().numpy()
        t0 = time.perf_counter()
        oracle.head_calibrate(q, k)
        dt += time.perf_counter() - t0
        n_h += 1
    return {"value": round(dt / n_h * H * 1e3, 1), "unit": "ms per call (estimated)",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d of %d heads (all %d sequences, full T=%d, d=%d) in %.1f s, scaled to %d heads"
                      % (n_h, H, N, T, d, dt, H)}


def rotate_timings(torch, saf, layers, steps, rounds=2):
    """Time each layer of `layers` (label -> Layer) for `steps` steps, in turn, `rounds` times, and
    keep each one's best round: (seconds per step, per-kernel summary).  Alternating keeps slow
    drifts of the clock from favouring whichever variant happens to run first."""
    best = {}
    for _ in range(rounds):
        for label, lv in layers.items():
            trace = saf.KernelTrace(capacity=4 * (steps + 1))
            tv = time_steps(torch, lv, steps, 2, trace)
            if label not in best or tv < best[label][0]:
                best[label] = (tv, trace.summary())
            trace.close()
    return best


def variants_of(torch, saf, w, dev, steps, mixed=None, draw_on=None):
    """The layer with all heads ordinary and with all heads replaced (same shape), timed in rotation
    with the mixed layer `mixed`: ordinary-tile efficiency, replaced vs ordinary time per head, and
    the mixed layer's speedup over all-ordinary (the analogue of the pages' speedup over ordinary
    attention).  Returns (variants, the mixed layer's best (seconds, kernel summary) or None)."""
    layers = {"all_ordinary": Layer(saf, torch, w, [0] * w.H, dev, draw_on=draw_on),
              "all_replaced": Layer(saf, torch, w, [1] * w.H, dev, draw_on=draw_on)}
    if mixed is not None:
        layers["mixed"] = mixed
    best = rotate_timings(torch, saf, layers, steps)
    var = {}
    for label, rr in (("all_ordinary", [0] * w.H), ("all_replaced", [1] * w.H)):
        tv, summ = best[label]
        fv = total_flops(w.B, w.T, w.d, rr, w.backward)
        var[label] = {"ms_per_step": round(tv * 1e3, 4), "tflops": round(fv / tv / 1e12, 1),
                      "pct_bf16_peak": round(100 * fv / tv / 1e12 / PEAK_BF16_TFLOPS, 2),
                      "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in summ.items()}}
    if mixed is not None:
        var["mixed_ms_per_step"] = round(best["mixed"][0] * 1e3, 4)
        var["mixed_speedup_vs_all_ordinary"] = round(best["all_ordinary"][0] / best["mixed"][0], 4)
    var["replaced_vs_ordinary_time_per_head"] = round(
        var["all_replaced"]["ms_per_step"] / var["all_ordinary"]["ms_per_step"], 4)
    var["timing"] = "best of 2 rounds, the variants%s timed in turn" % (" and the mixed layer" if mixed is not None else "")
    del layers
    return var, best.get("mixed")


def config_line(torch, saf, name, dev, steps):
    """One more workload of the pages' tables (inputs drawn on the GPU), timed in rotation with its
    all-ordinary / all-replaced variants (best of 2 rounds each): tokens/s, TFLOP/s, % of peak,
    per-kernel times and the variants."""
    import synth
    w = synth.WORKLOADS[name]
    rep = w.replaced()
    lay = Layer(saf, torch, w, rep, dev, draw_on="cuda")
    var, (t, summ) = variants_of(torch, saf, w, dev, steps, mixed=lay, draw_on="cuda")
    kf = kernel_flops(w.B, w.T, w.d, rep)
    kernels = {}
    for kname, st in summ.items():
        ent = {"avg_ms": round(st["avg_ms"], 4)}
        if kf.get(kname):
            ent["tflops"] = round(kf[kname] / (st["avg_ms"] * 1e-3) / 1e12, 1)
        kernels[kname] = ent
    del lay
    fl = total_flops(w.B, w.T, w.d, rep, w.backward)
    return {"workload": "%s: B=%d, H=%d, T=%d, d=%d, bf16, %d replaced, %s"
                        % (w.name, w.B, w.H, w.T, w.d, w.n_replaced, "fwd+bwd" if w.backward else "fwd"),
            "ms_per_step": round(t * 1e3, 4), "tokens_per_s": round(w.B * w.T / t, 1),
            "tflops": round(fl / t / 1e12, 1),
            "pct_bf16_peak": round(100 * fl / t / 1e12 / PEAK_BF16_TFLOPS, 2),
            "kernels": kernels,
            "variants": var}


CONFIGS = ["l124m_t4096", "l124m_t8192", "prefill_b64_t4096", "prefill_b2_t16384"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="l1b_t8192")
    ap.add_argument("--configs", default=",".join(CONFIGS),
                    help="comma-separated further workloads timed into the line's configs object")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--dq-recomputed", action="store_true",
                    help="time the headline layer with the smaller backward workspace (dQ forms S and "
                         "dP again) instead of the one that keeps dS")
    ap.add_argument("--no-pattern-grad", action="store_true")
    ap.add_argument("--no-latency", action="store_true")
    ap.add_argument("--calibration-workload", default="l1b_t8192",
                    help="workload whose calibration shape (N sequences) is timed")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device-to-device copies of MIB MiB (calibrates the HBM "
                         "byte counters of a profiler against a known size) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the layer has no exchange between GPUs, and a "
              "multi-GPU run is not provided (--gpus %d, WORLD_SIZE %d requested)"
              % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        n = args.copy_probe * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)
        return

    import fixed_pattern_mixed_amd as saf
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    replaced = w.replaced()
    layer = Layer(saf, torch, w, replaced, dev)
    layer.recompute_ds = args.dq_recomputed
    spin_ms, gemm_tflops = spin_up(torch)
    trace = saf.KernelTrace(capacity=4 * (args.steps + 1))
    per_step = []
    t_step = time_steps(torch, layer, args.steps, args.warmup, trace, per_step)
    tokens = w.B * w.T
    flops = total_flops(w.B, w.T, w.d, replaced, w.backward)
    kf = kernel_flops(w.B, w.T, w.d, replaced)

    kernels = {}
    for name, s in trace.summary().items():
        ent = {"avg_ms": round(s["avg_ms"], 4), "launches": s["launches"]}
        if kf.get(name):
            ent["tflops"] = round(kf[name] / (s["avg_ms"] * 1e-3) / 1e12, 1)
        kernels[name] = ent
    trace.close()
    dom = max(trace.summary().items(), key=lambda kv: kv[1]["total_ms"])[0]
    dom_ms = trace.summary()[dom]["avg_ms"]
    achieved = kf[dom] / (dom_ms * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(w.name, dom)}

    out = {
        "metric": METRIC,
        "value": round(tokens / t_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.kv_heads, "T": w.T, "d": w.d,
                   "replaced_heads": [h for h, x in enumerate(replaced) if x],
                   "pass": "fwd+bwd" if w.backward else "fwd",
                   "backward": ("dq_recomputed" if layer.recompute_ds or layer.nb == layer.nb_min
                                else "stored_ds") if w.backward else None,
                   "global_batch": w.B, "seq_len": w.T, "parallelism": "single-gpu"},
        "tflops": round(flops / t_step / 1e12, 1),
        "pct_bf16_peak": round(100 * flops / t_step / 1e12 / PEAK_BF16_TFLOPS, 2),
        "step_ms": step_spread(per_step),
        "kernels": kernels,
        "pattern_prepare_ms": round(layer.prepare_ms, 3),
        "gpu_spin_up_ms": spin_ms,
        "reference_gemm_tflops": gemm_tflops,
        "roofline": roofline,
        "backward": backward_unit(kernels, kf),
    }

    if not args.no_variants:
        var, _ = variants_of(torch, saf, w, dev, max(5, args.steps // 3), mixed=layer)
        if w.backward:  # the same layer with the backward's two kernels overlapped on two streams
            saf.saf_set_backward_overlap(1)
            to = time_steps(torch, layer, max(5, args.steps // 3), 2)
            saf.saf_set_backward_overlap(0)
            var["backward_overlap"] = {"ms_per_step": round(to * 1e3, 4),
                                       "tokens_per_s": round(tokens / to, 1)}
            if layer.nb > layer.nb_min:  # the backward with dQ re-forming S and dP (no stored dS)
                layer.recompute_ds = True
                tr = saf.KernelTrace(capacity=4 * (max(5, args.steps // 3) + 1))
                tq = time_steps(torch, layer, max(5, args.steps // 3), 2, tr)
                layer.recompute_ds = False
                var["dq_recomputed"] = {"ms_per_step": round(tq * 1e3, 4),
                                        "tokens_per_s": round(tokens / tq, 1),
                                        "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in tr.summary().items()}}
                tr.close()
        out["variants"] = var

    if not args.no_configs and args.configs:
        out["configs"] = {name: config_line(torch, saf, name, dev, max(5, args.steps // 2))
                          for name in args.configs.split(",") if name and name != w.name}

    if not args.no_pattern_grad:
        pg = pattern_gradient(torch, saf, layer, max(5, args.steps // 3))
        if pg is not None:
            pg["step_with_trainable_pattern_ms"] = round(t_step * 1e3 + pg["ms"], 4)
            out["trainable_pattern_gradient"] = pg

    if not args.no_latency:
        out["prefill_latency_b1"] = prefill_latency(torch, saf, dev)

    if not args.no_calibration:
        cw = synth.WORKLOADS[args.calibration_workload]
        if cw.calib_N:
            out["calibration"] = calibration(torch, saf, cw)
            if not args.no_cpu_baseline:
                out["calibration"]["cpu_baseline"] = cpu_calibration_baseline(cw)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, replaced)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
