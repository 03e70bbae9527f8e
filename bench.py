#!/usr/bin/env python3
"""Benchmark of the Q8_0 quantized matmul on one MI355X.

Headline (the single JSON line's `value`): the decode matvec workload
attn_q_b (in_dim 1024 -> out_dim 32768, n_tok 1).  One step = quantize the
fp32 activation row + the Q8_0 matmul, done by one fused launch
(q8_0_matmul_list); the same step as two calls (q8_0_quantize_act +
q8_0_matmul) is reported beside it.  value = algorithmic bytes of the step
(weights, fp32 row, fp32 output) / step time, in GB/s.
Inputs are resident in HBM before timing starts; the weights rotate through
16 independent copies (570 MB) so the 256 MB Infinity Cache cannot serve
them.

The same line also carries, under "secondary", the other workloads timed the
same way (decode5, router + shared expert gate/up, moe, prefill_a,
prefill_b) with their own roofline fractions; prefill reports int8 TOPS
against the int8 MFMA peak.

Options: --steps K --warmup W (headline loop), --gpus N (only 1 is
supported: this is a single-GPU path), --quick (headline only),
--calibrate (adds a plain device copy of known size for counter scaling),
--cpu-seconds S (time budget of the CPU-oracle baseline, 0 to skip).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
INT8_MFMA_PEAK_TOPS = 5000.0  # MI355X dense int8 matrix peak, TOPS
METRIC = "Q8_0 matmul GB/s at n_tok=1 & int8 TOPS at n_tok≥2048; % of roofline"
ROT = 16                      # weight copies rotated through in decode loops


def row_bytes(k):
    return k // 32 * 34


def profiled_traffic(profile):
    """HBM bytes per launch from the committed rocprofv3 byte-counter summary,
    or None when the kernel sources changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    h = re.search(r"source_sha256_16: ([0-9a-f]+)\s+\(([^)]*)\)", text)
    if not m or not h:
        return None
    digest = hashlib.sha256()
    for f in h.group(2).split(", "):
        digest.update(open(os.path.join(ROOT, f), "rb").read())
    return int(m.group(1)) if digest.hexdigest()[:16] == h.group(1) else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def capture(torch, fn, n):
    """A HIP graph of fn(0), ..., fn(n-1), captured on torch's capture stream
    (the library enqueues on torch's current stream, so its kernels land in
    the graph).  Eager warm-up first, so no first-call work is captured."""
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_steps(torch, fn, steps, warmup, per_graph=ROT):
    """Whole-step throughput: exactly `steps` steps, as replays of a graph
    holding `per_graph` consecutive steps fn(0..per_graph-1) plus one graph of
    the remaining steps, wall clock bracketed by synchronize.  `warmup`
    untimed steps run first, the same way."""
    steps = max(1, int(steps))
    per_graph = max(1, min(per_graph, steps))
    g = capture(torch, fn, per_graph)
    rest = steps % per_graph
    g_rest = capture(torch, fn, rest) if rest else None
    full = steps // per_graph
    for _ in range(-(-max(0, warmup) // per_graph)):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(full):
        g.replay()
    if g_rest is not None:
        g_rest.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) / steps, steps


def time_kernel(torch, fn, n_per_graph, reps=20):
    """Mean duration of one launch: HIP events on the current stream around
    replays of a graph of `n_per_graph` back-to-back launches of fn(i)."""
    g = capture(torch, fn, n_per_graph)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs)
    return 1000.0 * ms / (reps * n_per_graph)


def bench_attn_q_b(torch, q8, wl, steps, warmup):
    """One step = quantize the fp32 row + the Q8_0 matvec, as one fused launch
    (q8_0_matmul_list with the fp32 row).  The separate-call form of the same
    step (q8_0_quantize_act + q8_0_matmul) is timed beside it."""
    d = wl.attn_q_b("cuda")
    k, n = d["in_dim"], d["out_dim"]
    ws = [q8.q8_0_quantize_act(wl.attn_q_b("cuda", copy=c)["w"]) for c in range(ROT)]
    x = d["x"]
    xq = torch.empty((1, row_bytes(k)), dtype=torch.uint8, device="cuda")
    out = torch.empty((1, n), dtype=torch.float32, device="cuda")
    items = [[dict(out=out, w=ws[c], x=x, in_dim=k, out_dim=n)] for c in range(ROT)]

    def step(i):
        q8.q8_0_matmul_list(items[i % ROT], 1)

    def step_separate(i):
        q8.q8_0_quantize_act(x, out=xq)
        q8.q8_0_matmul(ws[i % ROT], xq, k, n, 1, out=out)

    sec, done = time_steps(torch, step, steps, warmup)
    sec_sep, _ = time_steps(torch, step_separate, steps, warmup)
    kern_us = time_kernel(torch, step, ROT)
    mv_us = time_kernel(torch, lambda i: q8.q8_0_matmul(ws[i % ROT], xq, k, n, 1, out=out), ROT)
    quant_us = time_kernel(torch, lambda i: q8.q8_0_quantize_act(x, out=xq), ROT)
    # Measured ceiling: a coalesced non-temporal streaming read of the same weight copies.
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    read_us = time_kernel(torch, lambda i: q8.q8_0_probe_read(ws[i % ROT], sink), ROT)
    # The fixed part of any launch: an empty kernel of 1024 workgroups, timed the same way.
    launch_us = time_kernel(torch, lambda i: q8.q8_0_probe_launch(1024, sink), ROT)
    fused_bytes = n * row_bytes(k) + 4 * k + 4 * n       # W + fp32 x + out
    mv_bytes = n * row_bytes(k) + row_bytes(k) + 4 * n   # W + x_q + out
    return dict(sec=sec, steps=done, step_bytes=fused_bytes, kernel_bytes=fused_bytes,
                kernel_us=kern_us, sec_separate=sec_sep, matvec_us=mv_us, matvec_bytes=mv_bytes,
                quant_us=quant_us, plan=q8.q8_0_matmul_plan(k, n, 1, 0),
                read_us=read_us, read_bytes=n * row_bytes(k), launch_us=launch_us)


def bench_decode5(torch, q8, wl, steps, warmup):
    """One step = the five decode projections of a layer from fp32 rows, as
    one q8_0_matmul_list call (the in_dim-32768 row is quantized by its own
    launch first; the other four are quantized inside the list launch)."""
    rot = 8
    sets = [wl.decode5("cuda", copy=c) for c in range(rot)]
    wq = [[q8.q8_0_quantize_act(p["w"]) for p in s] for s in sets]
    xs = [p["x"] for p in sets[0]]
    dims = [(p["in_dim"], p["out_dim"]) for p in sets[0]]
    xqs = [torch.empty((1, row_bytes(k)), dtype=torch.uint8, device="cuda") for k, _ in dims]
    outs = [torch.empty((1, n), dtype=torch.float32, device="cuda") for _, n in dims]
    del sets
    lists = [[dict(out=outs[j], w=wq[c][j], x=xs[j], x_q=xqs[j], in_dim=k, out_dim=n)
              for j, (k, n) in enumerate(dims)] for c in range(rot)]

    def step(i):
        q8.q8_0_matmul_list(lists[i % rot], 1)

    def step_separate(i):
        for j, (k, n) in enumerate(dims):
            q8.q8_0_quantize_act(xs[j], out=xqs[j])
            q8.q8_0_matmul(wq[i % rot][j], xqs[j], k, n, 1, out=outs[j])

    sec, done = time_steps(torch, step, steps, warmup, per_graph=rot)
    sec_sep, _ = time_steps(torch, step_separate, steps, warmup, per_graph=rot)

    # The five matmuls from x_q in one list launch, the quantizer reported
    # separately (five launches, one per x row).
    for j in range(len(dims)):
        q8.q8_0_quantize_act(xs[j], out=xqs[j])
    qlists = [[dict(out=outs[j], w=wq[c][j], x_q=xqs[j], in_dim=k, out_dim=n)
               for j, (k, n) in enumerate(dims)] for c in range(rot)]
    sec_xq, _ = time_steps(torch, lambda i: q8.q8_0_matmul_list(qlists[i % rot], 1), steps, warmup,
                           per_graph=rot)
    list_xq_us = time_kernel(torch, lambda i: q8.q8_0_matmul_list(qlists[i % rot], 1), rot)

    def quantize_all(i):
        for j in range(len(dims)):
            q8.q8_0_quantize_act(xs[j], out=xqs[j])

    quant_us = time_kernel(torch, quantize_all, rot)
    per = []
    for j, (k, n) in enumerate(dims):
        us = time_kernel(torch, lambda i, j=j, k=k, n=n: q8.q8_0_matmul(wq[i % rot][j], xqs[j], k, n, 1,
                                                                           out=outs[j]), rot)
        per.append(dict(name=wl.DECODE5[j][0], kernel_us=us,
                        kernel_bytes=n * row_bytes(k) + row_bytes(k) + 4 * n))
    w_bytes = sum(n * row_bytes(k) for k, n in dims)
    step_bytes = w_bytes + sum(4 * k + 4 * n for k, n in dims)  # W + fp32 x + out
    xq_bytes = w_bytes + sum(row_bytes(k) + 4 * n for k, n in dims)  # W + x_q + out
    return dict(sec=sec, sec_separate=sec_sep, step_bytes=step_bytes, w_bytes=w_bytes,
                per_matrix=per, sec_xq=sec_xq, list_xq_us=list_xq_us, xq_bytes=xq_bytes,
                quant_us=quant_us)


def bench_router_shared(torch, q8, wl, steps, warmup):
    """Decode router + shared expert gate/up from one fp32 row (4096): the
    router (ffn_gate_inp, 4096 -> 256) and the shared expert's gate and up
    (4096 -> 2048 each) as one q8_0_matmul_list launch."""
    rot = ROT
    k = 4096
    x = wl.normal((1, k), wl.X_STD, "cuda", "decode5", "ffn_gate_inp", "x")
    sets = []
    for c in range(rot):
        router = wl.normal((256, k), wl.W_STD, "cuda", "decode5", "ffn_gate_inp", "w", c)
        gate = wl.normal((2048, k), wl.W_STD, "cuda", "moe", "shared", -1, "gate", c)
        up = wl.normal((2048, k), wl.W_STD, "cuda", "moe", "shared", -1, "up", c)
        sets.append([q8.q8_0_quantize_act(t) for t in (router, gate, up)])
    dims = [(k, 256), (k, 2048), (k, 2048)]
    outs = [torch.empty((1, n), dtype=torch.float32, device="cuda") for _, n in dims]
    xq = torch.empty((1, row_bytes(k)), dtype=torch.uint8, device="cuda")
    lists = [[dict(out=outs[j], w=sets[c][j], x=x, in_dim=kk, out_dim=n)
              for j, (kk, n) in enumerate(dims)] for c in range(rot)]

    def step(i):
        q8.q8_0_matmul_list(lists[i % rot], 1)

    def step_separate(i):
        q8.q8_0_quantize_act(x, out=xq)
        for j, (kk, n) in enumerate(dims):
            q8.q8_0_matmul(sets[i % rot][j], xq, kk, n, 1, out=outs[j])

    sec, done = time_steps(torch, step, steps, warmup, per_graph=rot)
    sec_sep, _ = time_steps(torch, step_separate, steps, warmup, per_graph=rot)
    step_bytes = sum(n * row_bytes(kk) + 4 * n for kk, n in dims) + 4 * k
    return dict(sec=sec, sec_separate=sec_sep, step_bytes=step_bytes)


def bench_moe(torch, q8, wl, steps, warmup):
    cfg = wl.MOE
    E, kk, T, D, F = cfg["n_expert"], cfg["n_used"], cfg["n_tok"], cfg["d_model"], cfg["d_ff"]
    sel = wl.moe_routing().cuda()
    x, mid = wl.moe_acts("cuda")
    stacks, shared = {}, {}
    for which, (rows, cols) in (("gate", (F, D)), ("up", (F, D)), ("down", (D, F))):
        st = torch.empty((E, rows, row_bytes(cols)), dtype=torch.uint8, device="cuda")
        for e in range(E):
            q8.q8_0_quantize_act(wl.moe_expert(e, which, "cuda"), out=st[e])
        stacks[which] = st
        shared[which] = q8.q8_0_quantize_act(wl.moe_expert(-1, which, "cuda"))
    tables = {w: q8.expert_table(stacks[w]) for w in stacks}
    xq = torch.empty((T, row_bytes(D)), dtype=torch.uint8, device="cuda")
    midq = torch.empty((mid.shape[0], row_bytes(F)), dtype=torch.uint8, device="cuda")
    o_g = torch.empty((T, kk, F), device="cuda")
    o_u = torch.empty((T, kk, F), device="cuda")
    o_d = torch.empty((T, kk, D), device="cuda")
    s_g = torch.empty((T, F), device="cuda")
    s_u = torch.empty((T, F), device="cuda")
    s_d = torch.empty((T, D), device="cuda")
    wsm = torch.empty(q8.q8_0_moe_workspace_bytes(T, kk, E), dtype=torch.uint8, device="cuda")
    wsd = q8.matmul_workspace(D, F, T)
    wsd2 = q8.matmul_workspace(F, D, T)

    gate = lambda i: q8.q8_0_moe_grouped(tables["gate"], E, sel, xq, D, F, 0, out=o_g, workspace=wsm)
    down = lambda i: q8.q8_0_moe_grouped(tables["down"], E, sel, midq[:T * kk], F, D, 1, out=o_d,
                                          workspace=wsm)
    sh_gate = lambda i: q8.q8_0_matmul(shared["gate"], xq, D, F, T, out=s_g, workspace=wsd)

    def step(i):
        q8.q8_0_quantize_act(x, out=xq)
        gate(i)
        q8.q8_0_moe_grouped(tables["up"], E, sel, xq, D, F, 0, out=o_u, workspace=wsm)
        sh_gate(i)
        q8.q8_0_matmul(shared["up"], xq, D, F, T, out=s_u, workspace=wsd)
        q8.q8_0_quantize_act(mid, out=midq)
        down(i)
        q8.q8_0_matmul(shared["down"], midq[T * kk:], F, D, T, out=s_d, workspace=wsd2)

    sec, done = time_steps(torch, step, steps, warmup, per_graph=1)
    # One q8_0_moe_grouped call = routing kernel + grouped kernel; timed whole.
    gate_us = time_kernel(torch, gate, 1, reps=10)
    down_us = time_kernel(torch, down, 1, reps=10)
    sh_us = time_kernel(torch, sh_gate, 8, reps=5)
    # The routed FFN as one q8_0_moe_ffn call (route, gate+up with SwiGLU,
    # mid quantize, down, weighted combine) on the same x_q.
    route_w = torch.rand((T, kk), generator=torch.Generator().manual_seed(23)).cuda()
    f_out = torch.empty((T, D), device="cuda")
    wsf = torch.empty(q8.q8_0_moe_ffn_workspace_bytes(T, kk, E, D, F), dtype=torch.uint8,
                      device="cuda")
    ffn = lambda i: q8.q8_0_moe_ffn(tables["gate"], tables["up"], tables["down"], E, sel, route_w,
                                    xq, D, F, 0.0, out=f_out, workspace=wsf)
    ffn_us = time_kernel(torch, ffn, 1, reps=10)
    touched = int(torch.unique(sel).numel())
    mat = F * row_bytes(D)  # bytes of one expert matrix (gate/up/down are equal)
    pairs = T * kk
    gate_bytes = touched * mat + pairs * F * 4 + T * row_bytes(D)
    down_bytes = touched * mat + pairs * (row_bytes(F) + D * 4)
    g_bytes = 2 * gate_bytes + down_bytes
    s_bytes = 3 * mat + 2 * (T * F * 4 + T * row_bytes(D)) + T * (row_bytes(F) + D * 4)
    q_bytes = T * (4 * D + row_bytes(D)) + mid.shape[0] * (4 * F + row_bytes(F))
    ops = 2 * (pairs + T) * 3 * F * D
    ffn_bytes = 3 * touched * mat + T * row_bytes(D) + pairs * 8 + T * D * 4
    return dict(sec=sec, step_bytes=g_bytes + s_bytes + q_bytes, gate_us=gate_us, down_us=down_us,
                ffn_us=ffn_us, ffn_bytes=ffn_bytes,
                gate_bytes=gate_bytes, down_bytes=down_bytes, shared_us=sh_us,
                shared_bytes=mat + T * F * 4 + T * row_bytes(D), touched_experts=touched, ops=ops)


def probe_mfma_tops(torch, q8, mix=None):
    """Measured matrix-core ceilings, no memory traffic, in TOPS of int8 work:
    independent int8 MFMA chains (q8_0_probe_mfma_i8), or with `mix` the
    GEMM's whole per-tile-block instruction mix (q8_0_probe_mfma_mix: 1 =
    int8 + scale + unbias MFMAs and 16 fmas, the ceiling of the exact
    formulation as the kernel issues it; 2 = the int->float conversion on the
    VALU instead)."""
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    iters = 2000
    if mix is None:
        fn = lambda i: q8.q8_0_probe_mfma_i8(iters, sink)
    else:
        fn = lambda i: q8.q8_0_probe_mfma_mix(iters, mix, sink)
    us = time_kernel(torch, fn, 1, reps=5)
    return q8.PROBE_MFMA_OPS_PER_ITER * iters / (us * 1e-6) / 1e12


def bench_prefill(torch, q8, wl, name, steps, warmup):
    d = wl.prefill(name, "cuda")
    k, n, t = d["in_dim"], d["out_dim"], d["n_tok"]
    wq = q8.q8_0_quantize_act(d["w"])
    x = d["x"]
    del d
    xq = torch.empty((t, row_bytes(k)), dtype=torch.uint8, device="cuda")
    out = torch.empty((t, n), dtype=torch.float32, device="cuda")
    ws = q8.matmul_workspace(k, n, t)
    quant = lambda i: q8.q8_0_quantize_act(x, out=xq)
    gemm = lambda i: q8.q8_0_matmul(wq, xq, k, n, t, out=out, workspace=ws)

    def step(i):
        quant(i)
        gemm(i)

    sec, done = time_steps(torch, step, steps, warmup, per_graph=1)
    ops = 2 * t * n * k
    return dict(sec=sec, ops=ops, kernel_us=time_kernel(torch, gemm, 4, reps=5),
                quant_us=time_kernel(torch, quant, 4, reps=5),
                quant_bytes=t * (4 * k + row_bytes(k)),
                kernel_bytes=n * row_bytes(k) + t * row_bytes(k) + 4 * t * n,
                plan=q8.q8_0_matmul_plan(k, n, t, ws.numel()))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_cpu(fn, seconds):
    """Mean seconds per call of fn, repeated for about `seconds` (at least once)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    return (time.perf_counter() - t0) / reps, reps


def cpu_baseline(wl, seconds):
    """The oracle (plain C as committed) on every workload, on this host's CPU:
    once single-threaded and once on the host's cores (OpenMP over independent
    outputs, same results).  Each workload gets a bounded sample (stated),
    repeated for about seconds / 10 per thread setting, and is reported in the
    unit the GPU line uses for that workload.  Rates of a sample are its own
    algorithmic bytes (or operations) over its time."""
    import numpy as np
    import oracle

    threads = oracle.host_threads()
    per = max(0.2, seconds / 10.0)
    rows = []

    def measure(name, unit, work, sample, fn):
        res = {"workload": name, "unit": unit, "sample": sample}
        for th in (1, threads):
            with oracle.threads(th):
                sec, reps = _time_cpu(fn, per)
            res["single_thread" if th == 1 else "all_threads"] = round(work / sec / 1e9, 4)
            res["ms_single" if th == 1 else "ms_all"] = round(sec * 1e3, 3)
        res["threads"] = threads
        rows.append(res)

    # tiny: quantize both operands and multiply (the whole workload).
    d = wl.tiny("cpu")
    w, x = d["w"].numpy(), d["x"].numpy()
    measure("tiny", "GB/s", 128 * row_bytes(256) + 4 * row_bytes(256) + 4 * 128 * 4,
            "whole workload: quantize W and x, matmul 128x256 by 4 tokens",
            lambda: oracle.matmul(oracle.quantize(w), oracle.quantize(x), 256, want_mag=False))
    # attn_q_b: the whole decode step (quantize x + matvec 32768 x 1024).
    d = wl.attn_q_b("cpu")
    wq = oracle.quantize(d["w"].numpy())
    xa = d["x"].numpy()
    step = 32768 * row_bytes(1024) + 4 * 1024 + 4 * 32768
    measure("attn_q_b", "GB/s", step, "whole step: quantize 1x1024, matmul 32768x1024",
            lambda: oracle.matmul(wq, oracle.quantize(xa), 1024, want_mag=False))
    headline = rows[-1]
    del wq
    # decode5: the five projections from fp32 rows.
    ps = wl.decode5("cpu")
    qs = [(oracle.quantize(p["w"].numpy()), p["x"].numpy(), p["in_dim"]) for p in ps]
    step = sum(p["out_dim"] * row_bytes(p["in_dim"]) + 4 * p["in_dim"] + 4 * p["out_dim"] for p in ps)
    measure("decode5", "GB/s", step, "whole step: five projections, each quantize + matvec",
            lambda: [oracle.matmul(w_, oracle.quantize(x_), k_, want_mag=False) for w_, x_, k_ in qs])
    del qs, ps
    # moe: the gate, up and down projections of the pairs of the first 2
    # tokens (16 of 512 pairs); bytes as for the GPU line: each touched
    # expert matrix once, plus x_q, mid_q and the outputs.
    cfg = wl.MOE
    D, F, k = cfg["d_model"], cfg["d_ff"], cfg["n_used"]
    n_t = 2
    sel = np.ascontiguousarray(wl.moe_routing().numpy()[:n_t])
    x, mid = wl.moe_acts("cpu")
    experts = sorted(set(sel.reshape(-1).tolist()))
    mats = {}
    with oracle.threads(threads):
        xq = oracle.quantize(x.numpy()[:n_t])
        mq = oracle.quantize(mid.numpy()[:n_t * k])
        for which in ("gate", "up", "down"):
            lst = [np.zeros((1, 34), np.uint8)] * cfg["n_expert"]
            for e in experts:
                lst[e] = oracle.quantize(wl.moe_expert(e, which, "cpu").numpy())
            mats[which] = lst
    pairs = n_t * k
    mat = F * row_bytes(D)
    work = (3 * len(experts) * mat + n_t * row_bytes(D) + 2 * pairs * F * 4
            + pairs * (row_bytes(F) + 4 * D))
    measure("moe", "GB/s", work,
            f"gate, up and down of the {pairs} (token, slot) pairs of tokens 0..{n_t - 1} "
            f"({len(experts)} experts)",
            lambda: [oracle.moe_grouped(mats["gate"], sel, xq, D, F, 0, want_mag=False),
                     oracle.moe_grouped(mats["up"], sel, xq, D, F, 0, want_mag=False),
                     oracle.moe_grouped(mats["down"], sel, mq, F, D, 1, want_mag=False)])
    del mats
    # prefill: 64 tokens x 256 output rows of each GEMM, whole K (TOPS).
    for name in ("prefill_a", "prefill_b"):
        d = wl.prefill(name, "cpu", rows=256, tokens=64)
        kk = d["in_dim"]
        wq = oracle.quantize(d["w"].numpy())
        xq = oracle.quantize(d["x"].numpy())
        measure(name, "TOPS", 2.0 * 64 * 256 * kk / 1e3,
                f"64 tokens x 256 output rows, whole K = {kk} (operands quantized beforehand)",
                lambda: oracle.matmul(wq, xq, kk, want_mag=False))
        del wq, xq, d
    return dict(value=headline["all_threads"], unit="GB/s", cores=threads, kind="oracle",
                sample=f"attn_q_b whole step (quantize 1x1024 + matvec 32768x1024) on {threads} "
                       f"threads: {headline['ms_all']} ms/step (single thread "
                       f"{headline['single_thread']} GB/s, {headline['ms_single']} ms/step); "
                       f"per_config has every workload",
                cpu_model=_cpu_model(), nproc=os.cpu_count(), threads_used=threads,
                per_config=rows)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--quick", action="store_true")
    ap.add_argument("--calibrate", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this Q8_0 path runs on exactly one GPU; --gpus must be 1 "
              "(multi-GPU sharding is described in DESIGN.md, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import q8_quantized_matmul_amd as q8
    import workloads as wl
    torch.cuda.set_device(0)

    if args.calibrate:
        # A plain device-to-device copy of 1 GiB, for scaling HBM byte counters.
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    log("[bench] attn_q_b")
    h = bench_attn_q_b(torch, q8, wl, args.steps, args.warmup)
    value = h["step_bytes"] / h["sec"] / 1e9
    ach = h["kernel_bytes"] / (h["kernel_us"] * 1e-6) / 1e9
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": h["steps"], "warmup": args.warmup, "ms_per_step": round(h["sec"] * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "attn_q_b decode: fp32 x[1x1024] quantized to Q8_0 and multiplied by "
                               "Q8_0 W[32768x1024] -> fp32, one fused launch per step "
                               "(q8_0_matmul_list), 16 rotating weight copies",
                   "in_dim": 1024, "out_dim": 32768, "n_tok": 1, "kernel_plan": list(h["plan"])},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "measured_ceiling": {
                         "kind": "coalesced non-temporal streaming read of the same weight copies (q8_0_probe_read)",
                         "GBs": round(h["read_bytes"] / (h["read_us"] * 1e-6) / 1e9, 1),
                         "frac": round(ach / (h["read_bytes"] / (h["read_us"] * 1e-6) / 1e9), 4),
                         "read_us": round(h["read_us"], 3),
                         "launch_floor_us": round(h["launch_us"], 3),
                         "launch_floor_kind": "empty kernel, 1024 workgroups (q8_0_probe_launch)"},
                     "traffic": profiled_traffic("matvec_list_attn_q_b.md"),
                     "kernel": "matvec_fused_kernel (the one-item q8_0_matmul_list launch: in-launch quantize + matvec)",
                     "kernel_us": round(h["kernel_us"], 3), "bytes_per_launch": h["kernel_bytes"]},
        "separate_calls": {
            "ms_per_step": round(h["sec_separate"] * 1e3, 5),
            "GBs": round(h["matvec_bytes"] / h["sec_separate"] / 1e9, 1),
            "matvec_kernel_us": round(h["matvec_us"], 3),
            "matvec_kernel_GBs": round(h["matvec_bytes"] / (h["matvec_us"] * 1e-6) / 1e9, 1),
            "quantize_us": round(h["quant_us"], 3)},
    }
    secondary = []
    if not args.quick:
        log("[bench] decode5")
        d5 = bench_decode5(torch, q8, wl, max(args.steps // 2, 16), args.warmup)
        secondary.append({
            "workload": "decode5 (5 projections of a layer from fp32 rows, n_tok 1, one list call)",
            "value": round(d5["step_bytes"] / d5["sec"] / 1e9, 2), "unit": "GB/s",
            "ms_per_step": round(d5["sec"] * 1e3, 5),
            "frac_hbm": round(d5["step_bytes"] / d5["sec"] / 1e9 / HBM_PEAK_GBS, 4),
            "separate_calls_ms_per_step": round(d5["sec_separate"] * 1e3, 5),
            "from_x_q": {
                "what": "the five matmuls from x_q in one list launch (quantizer below, separately)",
                "GBs": round(d5["xq_bytes"] / d5["sec_xq"] / 1e9, 1),
                "ms_per_step": round(d5["sec_xq"] * 1e3, 5),
                "frac_hbm": round(d5["xq_bytes"] / d5["sec_xq"] / 1e9 / HBM_PEAK_GBS, 4),
                "list_kernel_us": round(d5["list_xq_us"], 3),
                "list_kernel_frac_hbm": round(d5["xq_bytes"] / (d5["list_xq_us"] * 1e-6) / 1e9
                                              / HBM_PEAK_GBS, 4),
                "bytes": d5["xq_bytes"],
                "quantize_five_rows_us": round(d5["quant_us"], 3)},
            "per_matrix_q8_0_matmul": [
                {"name": p["name"], "kernel_us": round(p["kernel_us"], 3),
                 "GBs": round(p["kernel_bytes"] / (p["kernel_us"] * 1e-6) / 1e9, 1)}
                for p in d5["per_matrix"]]})
        log("[bench] router_shared")
        rs = bench_router_shared(torch, q8, wl, max(args.steps // 2, 16), args.warmup)
        secondary.append({
            "workload": "router + shared expert gate/up (4096 -> 256, 2048, 2048) from one fp32 row, "
                        "one fused list launch",
            "value": round(rs["step_bytes"] / rs["sec"] / 1e9, 2), "unit": "GB/s",
            "ms_per_step": round(rs["sec"] * 1e3, 5),
            "frac_hbm": round(rs["step_bytes"] / rs["sec"] / 1e9 / HBM_PEAK_GBS, 4),
            "separate_calls_ms_per_step": round(rs["sec_separate"] * 1e3, 5)})
        log("[bench] moe")
        mo = bench_moe(torch, q8, wl, max(args.steps // 50, 5), 3)
        gate_gbs = mo["gate_bytes"] / (mo["gate_us"] * 1e-6) / 1e9
        secondary.append({
            "workload": "moe (64 tokens x 8 of 256 experts + shared, gate/up/down)",
            "value": round(mo["step_bytes"] / mo["sec"] / 1e9, 2), "unit": "GB/s",
            "ms_per_step": round(mo["sec"] * 1e3, 4), "touched_experts": mo["touched_experts"],
            "grouped_gate_us": round(mo["gate_us"], 2), "grouped_gate_GBs": round(gate_gbs, 1),
            "frac_hbm_grouped_gate": round(gate_gbs / HBM_PEAK_GBS, 4),
            "grouped_down_us": round(mo["down_us"], 2),
            "grouped_down_GBs": round(mo["down_bytes"] / (mo["down_us"] * 1e-6) / 1e9, 1),
            "shared_gate_us": round(mo["shared_us"], 2),
            "shared_gate_GBs": round(mo["shared_bytes"] / (mo["shared_us"] * 1e-6) / 1e9, 1),
            "routed_ffn_us": round(mo["ffn_us"], 2),
            "routed_ffn_GBs": round(mo["ffn_bytes"] / (mo["ffn_us"] * 1e-6) / 1e9, 1),
            "frac_hbm_routed_ffn": round(mo["ffn_bytes"] / (mo["ffn_us"] * 1e-6) / 1e9
                                         / HBM_PEAK_GBS, 4)})
        log("[bench] int8 MFMA probes")
        mfma_tops = probe_mfma_tops(torch, q8)
        mix_tops = probe_mfma_tops(torch, q8, mix=1)
        mix_valu_tops = probe_mfma_tops(torch, q8, mix=2)
        for name in ("prefill_a", "prefill_b"):
            log(f"[bench] {name}")
            pf = bench_prefill(torch, q8, wl, name, max(args.steps // 40, 10), 3)
            tops = pf["ops"] / (pf["kernel_us"] * 1e-6) / 1e12
            secondary.append({
                "workload": name, "value": round(pf["ops"] / pf["sec"] / 1e12, 2), "unit": "TOPS",
                "ms_per_step": round(pf["sec"] * 1e3, 4), "gemm_kernel_us": round(pf["kernel_us"], 2),
                "gemm_TOPS": round(tops, 1), "frac_int8_mfma": round(tops / INT8_MFMA_PEAK_TOPS, 4),
                "measured_mfma_TOPS": round(mfma_tops, 1),
                "frac_of_measured_mfma": round(tops / mfma_tops, 4),
                "formulation_ceiling_TOPS": round(mix_tops, 1),
                "frac_of_formulation_ceiling": round(tops / mix_tops, 4),
                "formulation_ceiling_valu_convert_TOPS": round(mix_valu_tops, 1),
                "quantize_us": round(pf["quant_us"], 2),
                "quantize_GBs": round(pf["quant_bytes"] / (pf["quant_us"] * 1e-6) / 1e9, 1),
                "plan": list(pf["plan"])})
    result["secondary"] = secondary
    if args.cpu_seconds > 0:
        log("[bench] cpu baseline")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
