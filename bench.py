#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 linear hot path on one MI355X.

Headline (the `value` of the JSON line): the LLaMA-65B-shaped full weight set,
80 layers x (q, k, v, o, gate, up, down) = 560 frozen NF4 + double-quant
linears resident in HBM (hidden 8192, MLP 22016), each with a rank-64 LoRA
adapter (alpha 16).  A step is the forward of all 560 linears in layer order
followed by the backward of all 560 in reverse order, at 512 tokens, every
linear on its own seeded synthetic input (nothing between the linears).
`value` is the algorithmic fwd+bwd rate, sum over linears of
4 T N K + 6 T r (K + N) flop per step, divided by the host wall time of
exactly --steps steps bracketed by device synchronisations.  Before the steps
the whole set is quantized on the device ("quantize_all": fp32 weights drawn
per layer, 3.2 GB a layer, every launch reading cold HBM), which is timed by
HIP events around the quantization kernels alone.

Beside it, in the same JSON line:
  roofline      the dominant kernel's algorithmic rate against the MI355X
                peak, from HIP events recorded on its launch stream during a
                second pass of the same steps;
  workloads     the LLaMA-33B decoder-layer linears (T=4096) and the
                LLaMA-7B MLP (T=2048), each with its own rate and roofline;
  gemv          the small-token forward (4096x4096, 4 tokens, r=64) over 48
                rotating weight copies (> 390 MB of codes: cold HBM);
  quantize      11008x4096 weights (fp32 and bf16) over 40 rotating source
                copies, median per-launch event time;
  gemv_grouped  the seven linears of a LLaMA-7B layer in one grouped
                small-token call (4 tokens), rotating over 4 layer copies;
  optimizer     AdamW with clipping over all 800 M adapter parameters of the
                65B set (state in HBM) and, paged, over one layer's (state in
                pinned host memory);
  peaks         the copy and bf16-MFMA rates this GPU sustains (probes), with
                the headline fractions against them;
  cpu_baseline  the CPU oracle on a bounded sample, per stage, median of 3.

    python bench.py [--steps K] [--warmup W] [--workload full65b|layer33b|mlp7b|tiny]
                    [--no-extras] [--no-cpu-baseline] [--legs workloads,gemv,...]

q, k, v and gate, up (same shape, the same input in a LLaMA block) run as
batched launches, the other linears alone; each linear keeps its own inputs
and outputs.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # HBM3E
METRIC = "QLoRA NF4 linear fwd+bwd TFLOP/s and dequant-GEMV GB/s, % of MI355X roofline"


def fwdbwd_flops(T, N, K, r):
    return 4 * T * N * K + 6 * T * r * (K + N)


def kernel_flops(name, T, N, K, r):
    """Algorithmic flops of one launch of the named kernel for one linear."""
    if name == "gemm_fwd_kernel":
        return 2 * T * N * K + 2 * T * r * N
    if name == "gemm_dx_kernel":
        return 2 * T * N * K + 2 * T * r * K
    return None


def dq_bytes(N, K):
    nb = N * K // 64
    return N * K // 2 + nb + 4 * ((nb + 255) // 256)


def gemv_kernel_bytes(T, N, K, r):
    """Algorithmic HBM bytes of one dequant-GEMV launch: codes, 8-bit and
    fp32 second-level constants, X, B, XA in and Y out, each once."""
    return dq_bytes(N, K) + 2 * T * K + 2 * r * N + 4 * T * r + 2 * T * N


def gemv_path_bytes(T, N, K, r):
    """Bytes of the whole small-token forward: the GEMV's plus A."""
    return gemv_kernel_bytes(T, N, K, r) - 4 * T * r + 2 * K * r


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_nf4_quantized_21_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 counters, if the committed
    measurement was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(*rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


def median(xs):
    return statistics.median(xs)


# ---------------------------------------------------------------------------
# Workload set-up: quantized weights resident in HBM plus per-linear inputs.
# ---------------------------------------------------------------------------
def linear_list(wl):
    """(seed index, name, N, K) of every linear of the workload, layer-major."""
    out = []
    for layer in range(wl.layers):
        for j, lin in enumerate(wl.linears):
            out.append((layer * len(wl.linears) + j, lin.name, lin.N, lin.K))
    return out


def quantize_all(torch, qlora, synth, wl, lins):
    """Quantize every linear of the workload from fp32 weights drawn on the
    device one layer at a time (one layer's fp32 set is generated, then its
    linears are quantized in generation order, so each read is from cold
    HBM), and time the quantization kernels with HIP events."""
    per_layer = len(wl.linears)
    layer_elems = sum(l.N * l.K for l in wl.linears)
    buf = torch.empty(layer_elems, dtype=torch.float32, device="cuda")
    weights = []
    qlora.timing_read()
    for layer in range(wl.layers):
        chunk = lins[layer * per_layer:(layer + 1) * per_layer]
        views, off = [], 0
        for (i, _, N, K) in chunk:
            v = buf[off:off + N * K]
            synth.device_weight(v, i)
            views.append(v)
            off += N * K
        qlora.timing_enable(True)
        for (i, _, N, K), v in zip(chunk, views):
            n = N * K
            codes = torch.empty(n // 2, dtype=torch.uint8, device="cuda")
            q8 = torch.empty(n // 64, dtype=torch.uint8, device="cuda")
            s2 = torch.empty((n // 64 + 255) // 256, dtype=torch.float32, device="cuda")
            qlora.quantize_dq(v, "nf4", codes, q8, s2)   # quantize + double quant in one pass
            weights.append((codes, q8, s2))
        qlora.timing_enable(False)
    torch.cuda.synchronize()
    kt = qlora.timing_read()
    del buf
    torch.cuda.empty_cache()
    params = sum(N * K for (_, _, N, K) in lins)
    ms = sum(t for (_, t) in kt.values())
    # algorithmic bytes of the one-pass kernel: fp32 weights read once;
    # codes, q8 and s2 written once
    nb = params // 64
    alg = 4 * params + params // 2 + nb + 4 * ((nb + 255) // 256)
    res = {"workload": f"{wl.name}: quantize all {len(lins)} linears from fp32 (blockwise NF4 + double quant in "
                       "one pass)",
           "params": params, "kernel_ms": round(ms, 3),
           "kernels": {k: {"launches": n, "total_ms": round(t, 3)} for k, (n, t) in kt.items()},
           "algorithmic_bytes": alg, "GBs": round(alg / (ms * 1e-3) / 1e9, 1),
           "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "note": "fp32 source drawn on the device per layer (3.2 GB) and never resident as a whole; "
                   "only the quantization kernels are timed"}
    return weights, res


# Linears of a layer that take the same input in a LLaMA block and have the
# same shape run as one batched launch (the layer's other linears alone).
FUSED_SETS = ({"q_proj", "k_proj", "v_proj"}, {"gate_proj", "up_proj"})


def make_linears(torch, qlora, synth, wl, lins, weights):
    """Per-linear inputs and gradients; shared Y / dX outputs and workspaces;
    `groups`: the launch groups of the step in layer order."""
    T, r = wl.T, wl.r
    Ls = []
    for (i, name, N, K), (codes, q8, s2) in zip(lins, weights):
        inp = synth.device_inputs(T, N, K, r, i, backward=True, weight=False)
        L = dict(T=T, N=N, K=K, r=r, name=name, codes=codes, q8=q8, s2=s2, **inp)
        L["XA"] = torch.empty(T, r, dtype=torch.float32, device="cuda")
        L["dA"] = torch.empty(K, r, dtype=torch.bfloat16, device="cuda")
        L["dB"] = torch.empty(r, N, dtype=torch.bfloat16, device="cuda")
        Ls.append(L)
    # batched launches write their linears' outputs at once: one Y / dX
    # buffer per member position of a group
    groups, cur = [], []
    for L in Ls:
        if cur and any(L["name"] in fs and cur[0]["name"] in fs for fs in FUSED_SETS) and \
                (L["N"], L["K"]) == (cur[0]["N"], cur[0]["K"]):
            cur.append(L)
        else:
            if cur:
                groups.append(cur)
            cur = [L]
    groups.append(cur)
    width = max(len(g) for g in groups)
    maxN = max(L["N"] for L in Ls)
    maxK = max(L["K"] for L in Ls)
    Ybuf = [torch.empty(T * maxN, dtype=torch.bfloat16, device="cuda") for _ in range(width)]
    dXbuf = [torch.empty(T * maxK, dtype=torch.bfloat16, device="cuda") for _ in range(width)]
    shapes = {tuple((L["K"], L["N"]) for L in g) for g in groups}
    wsf = wsb = 0
    for sh in shapes:
        if len(sh) == 1:   # a single linear runs through linear_fwd / linear_bwd
            (K, N), = sh
            wsf = max(wsf, qlora.linear_fwd_workspace_bytes(T, K, N, r))
            wsb = max(wsb, qlora.linear_bwd_workspace_bytes(T, K, N, r))
        else:
            wsf = max(wsf, qlora.grouped_workspace_bytes(list(sh), T, r))
            wsb = max(wsb, qlora.grouped_workspace_bytes(list(sh), T, r, backward=True))
    wsf = torch.empty(max(1, wsf), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(1, wsb), dtype=torch.uint8, device="cuda")
    for g in groups:
        for j, L in enumerate(g):
            L["Y"] = Ybuf[j][: T * L["N"]].view(T, L["N"])
            L["dX"] = dXbuf[j][: T * L["K"]].view(T, L["K"])
            L["wsf"], L["wsb"] = wsf, wsb
    return Ls, groups


def run_fwd(qlora, L, alpha):
    qlora.linear_fwd(L["X"], L["codes"], L["q8"], L["s2"], L["A"], L["B"], alpha, L["N"], Y=L["Y"], XA=L["XA"],
                     workspace=L["wsf"])


def run_bwd(qlora, L, alpha):
    qlora.linear_bwd(L["dY"], L["X"], L["XA"], L["codes"], L["q8"], L["s2"], L["A"], L["B"], alpha, dX=L["dX"],
                     dA=L["dA"], dB=L["dB"], workspace=L["wsb"])


def run_group_fwd(qlora, g, alpha):
    if len(g) == 1:
        run_fwd(qlora, g[0], alpha)
    else:
        qlora.linear_fwd_grouped(g, alpha, g[0]["T"], g[0]["r"], workspace=g[0]["wsf"])


def run_group_bwd(qlora, g, alpha):
    if len(g) == 1:
        run_bwd(qlora, g[0], alpha)
    else:
        qlora.linear_bwd_grouped(g, alpha, g[0]["T"], g[0]["r"], workspace=g[0]["wsb"])


def time_steps(torch, qlora, wl, Ls, groups, steps, warmup, event_steps):
    """Wall time per step of the fwd (layer order) + bwd (reverse order) step,
    then per-kernel event times from a second pass of event_steps steps."""
    alpha = wl.alpha

    def step():
        for g in groups:
            run_group_fwd(qlora, g, alpha)
        for g in reversed(groups):
            run_group_bwd(qlora, g, alpha)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    qlora.device_status()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    # second pass: every library kernel bracketed by events on its stream
    qlora.timing_read()
    qlora.timing_enable(True)
    t2 = time.perf_counter()
    for _ in range(event_steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    qlora.timing_enable(False)
    kt = qlora.timing_read()
    qlora.device_status()   # raises if a split hand-off wait ever ran out
    flops = sum(fwdbwd_flops(L["T"], L["N"], L["K"], L["r"]) for L in Ls)
    name, (launches, total_ms) = max(kt.items(), key=lambda kv: kv[1][1])
    per_step = [kernel_flops(name, L["T"], L["N"], L["K"], L["r"]) for L in Ls]
    roof = None
    if all(f is not None for f in per_step):
        achieved = sum(per_step) * event_steps / (total_ms * 1e-3) / 1e12
        launches_per_step = launches // event_steps
        roof = {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_from_profiles(name, WORKLOAD_TAG.get(wl.name, wl.name)),
                "avg_launch_us": round(total_ms * 1e3 / launches, 2), "launches": launches,
                "algorithmic_flop_per_launch": round(sum(per_step) / launches_per_step),
                "events_pass_ms_per_step": round((t3 - t2) * 1e3 / event_steps, 4)}
    tot = sum(v[1] for v in kt.values())
    kernels = {k: {"launches": n, "avg_us": round(t * 1e3 / n, 2), "share": round(t / tot, 4)}
               for k, (n, t) in sorted(kt.items(), key=lambda kv: -kv[1][1])}
    return ms, flops, roof, kernels


WORKLOAD_TAG = {"llama65b-80layers-T512-r64": "full65b", "llama33b-layer-T4096-r64": "layer33b",
                "llama7b-mlp-T2048-r64": "mlp7b", "tiny-512x512-T32-r8": "tiny"}


def bench_workload(torch, qlora, synth, key, steps, warmup, event_steps=2):
    wl = synth.WORKLOADS[key]
    lins = linear_list(wl)
    weights, qres = quantize_all(torch, qlora, synth, wl, lins)
    Ls, groups = make_linears(torch, qlora, synth, wl, lins, weights)
    del weights
    ms, flops, roof, kernels = time_steps(torch, qlora, wl, Ls, groups, steps, warmup, event_steps)
    value = flops / (ms * 1e-3) / 1e12
    res = {"workload": wl.name, "tokens": wl.T, "r": wl.r, "alpha": wl.alpha, "layers": wl.layers,
           "launch_groups": [[L["name"] for L in g] for g in groups[:len(wl.linears)]],
           "linears": [[l.name, l.N, l.K] for l in wl.linears], "flop_per_step": flops,
           "value": round(value, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 4), "steps": steps,
           "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4), "roofline": roof, "kernels": kernels,
           "quantize_all": qres}
    del Ls, groups
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# Small-token forward (dequant-GEMV) and quantization throughput, cold HBM.
# ---------------------------------------------------------------------------
def bench_gemv(torch, qlora, synth, copies=48, iters=240):
    T, N, K, r, alpha = 4, 4096, 4096, 64, 16.0
    lins = [(i, "q_proj", N, K) for i in range(copies)]
    Ls = []
    for (i, _, n_, k_) in lins:
        inp = synth.device_inputs(T, n_, k_, r, i, backward=False)
        codes, absmax = qlora.quantize_nf4(inp.pop("W").view(-1))
        q8, s2 = qlora.double_quant(absmax)
        L = dict(T=T, N=N, K=K, r=r, codes=codes, q8=q8, s2=s2, **inp)
        Ls.append(L)
    X = Ls[0]["X"]
    Y = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    XA = torch.empty(T, r, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, qlora.linear_fwd_workspace_bytes(T, K, N, r)), dtype=torch.uint8, device="cuda")
    for L in Ls:
        L.update(X=X, Y=Y, XA=XA, wsf=ws)
    for i in range(2 * copies):
        run_fwd(qlora, Ls[i % copies], alpha)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(iters):
        run_fwd(qlora, Ls[i % copies], alpha)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    qlora.timing_read()
    qlora.timing_enable(True)
    for i in range(iters):
        run_fwd(qlora, Ls[i % copies], alpha)
    torch.cuda.synchronize()
    qlora.timing_enable(False)
    kt = qlora.timing_read()
    n, total = kt["gemv_fwd_kernel"]
    us = total * 1e3 / n
    kb = gemv_kernel_bytes(T, N, K, r)
    gbs = kb / (us * 1e-6) / 1e9
    fwd_us = sum(t for (_, t) in kt.values()) * 1e3 / iters
    res = {"workload": "llama7b-q_proj-gemv-T4-r64 (4096x4096 NF4+DQ, 4 tokens, fwd)",
           "value": round(gbs, 1), "unit": "GB/s",
           "roofline": {"kernel": "gemv_fwd_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": traffic_from_profiles("gemv_fwd_kernel", "gemv7b"),
                        "avg_launch_us": round(us, 3), "bytes_per_launch": kb},
           "fwd_path_us_gpu": round(fwd_us, 3),
           "fwd_path_GBs_gpu": round(gemv_path_bytes(T, N, K, r) / (fwd_us * 1e-6) / 1e9, 1),
           "fwd_call_us_wall": round((t1 - t0) * 1e6 / iters, 3),
           "kernels_avg_us": {k: round(t * 1e3 / c, 3) for k, (c, t) in kt.items()},
           "weight_copies": copies, "codes_bytes_rotated": copies * dq_bytes(N, K)}
    del Ls
    torch.cuda.empty_cache()
    return res


def bench_gemv_grouped(torch, qlora, synth, copies=4, iters=40, T=4):
    """The grouped small-token forward over all seven linears of a LLaMA-7B
    layer (q, k, v, o 4096x4096; gate, up 4096->11008; down 11008->4096; 4
    tokens, r=64) in one call, rotating over 4 layer copies (415 MB of codes,
    cold HBM)."""
    r, alpha = 64, 16.0
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
    groups = []
    for c in range(copies):
        layer = []
        for j, (N, K) in enumerate(shapes):
            i = 7 * c + j
            W = torch.empty(N * K, dtype=torch.float32, device="cuda")
            synth.device_weight(W, i)
            codes, q8, s2 = qlora.quantize_dq(W)
            del W
            inp = synth.device_inputs(T, N, K, r, i, backward=False, weight=False)
            layer.append(dict(X=inp["X"], A=inp["A"], B=inp["B"], codes=codes, q8=q8, s2=s2,
                              Y=torch.empty(T, N, dtype=torch.bfloat16, device="cuda"),
                              XA=torch.empty(T, r, dtype=torch.float32, device="cuda")))
        groups.append(layer)
    ws = None
    for g in groups * 2:
        qlora.linear_fwd_grouped(g, alpha, T, r, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(iters):
        qlora.linear_fwd_grouped(groups[i % copies], alpha, T, r)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    qlora.timing_read()
    qlora.timing_enable(True)
    for i in range(iters):
        qlora.linear_fwd_grouped(groups[i % copies], alpha, T, r)
    torch.cuda.synchronize()
    qlora.timing_enable(False)
    kt = qlora.timing_read()
    n, total = kt["gemv_fwd_kernel"]
    us = total * 1e3 / n
    kb = sum(gemv_kernel_bytes(T, N, K, r) for (N, K) in shapes)
    gbs = kb / (us * 1e-6) / 1e9
    path_us = sum(t for (_, t) in kt.values()) * 1e3 / iters
    path_bytes = sum(gemv_path_bytes(T, N, K, r) for (N, K) in shapes)
    res = {"workload": f"llama7b-layer-grouped-gemv-T{T}-r64 (7 linears, 202M NF4+DQ weights, one call)",
           "value": round(gbs, 1), "unit": "GB/s",
           "roofline": {"kernel": "gemv_fwd_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "avg_launch_us": round(us, 3), "bytes_per_launch": kb},
           "fwd_path_us_gpu": round(path_us, 3),
           "fwd_path_GBs_gpu": round(path_bytes / (path_us * 1e-6) / 1e9, 1),
           "call_us_wall": round((t1 - t0) * 1e6 / iters, 3),
           "kernels_avg_us": {k: round(t * 1e3 / c, 3) for k, (c, t) in kt.items()},
           "layer_copies": copies, "codes_bytes_rotated": copies * sum(dq_bytes(N, K) for (N, K) in shapes)}
    del groups
    torch.cuda.empty_cache()
    return res


def _event_median(torch, fn, items, reps):
    """Median over reps calls of fn(item) (items rotated) of the per-call
    event time on the current stream, in microseconds."""
    times = []
    s = torch.cuda.current_stream()
    for k in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn(items[k % len(items)])
        b.record(s)
        times.append((a, b))
    torch.cuda.synchronize()
    return median([a.elapsed_time(b) * 1e3 for (a, b) in times])


def bench_quantize(torch, qlora, copies=40, reps=80):
    """Quantization of 11008 x 4096 weights, 40 distinct source copies (7.2 GB
    fp32, 3.6 GB bf16) rotated so every launch reads cold HBM; median of the
    per-launch event times."""
    N, K = 11008, 4096
    n = N * K
    nb = n // 64
    codes = torch.empty(n // 2, dtype=torch.uint8, device="cuda")
    absmax = torch.empty(nb, dtype=torch.float32, device="cuda")
    q8 = torch.empty(nb, dtype=torch.uint8, device="cuda")
    s2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device="cuda")
    from bit_nf4_quantized_21_amd import synth
    srcs = [synth.device_weight(torch.empty(n, dtype=torch.float32, device="cuda"), i) for i in range(copies)]
    absmaxes = [qlora.quantize_nf4(x, codes)[1] for x in srcs[:8]]
    for x in srcs:
        qlora.quantize_nf4(x, codes, absmax)
    q_us = _event_median(torch, lambda x: qlora.quantize_nf4(x, codes, absmax), srcs, reps)
    d_us = _event_median(torch, lambda a: qlora.double_quant(a, q8, s2), absmaxes, reps)
    f_us = _event_median(torch, lambda x: qlora.quantize_dq(x, "nf4", codes, q8, s2), srcs, reps)
    types = {}
    for kind in ("int4", "fp4"):
        t_us = _event_median(torch, lambda x: qlora.quantize_dq(x, kind, codes, q8, s2), srcs, reps)
        fb = 4 * n + n // 2 + nb + 4 * ((nb + 255) // 256)
        types[kind] = {"median_us": round(t_us, 2), "GBs": round(fb / (t_us * 1e-6) / 1e9, 1),
                       "frac_hbm": round(fb / (t_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    qbytes = 4 * n + n // 2 + 4 * nb
    dbytes = 4 * nb + nb + 4 * ((nb + 255) // 256)
    res = {"workload": "quantize 11008x4096 -> NF4 + double quant, 40 rotating source copies",
           "source_bytes_rotated": copies * 4 * n,
           "quantize_fp32": {"median_us": round(q_us, 2), "GBs": round(qbytes / (q_us * 1e-6) / 1e9, 1),
                             "frac_hbm": round(qbytes / (q_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "bytes": qbytes},
           "double_quant": {"median_us": round(d_us, 2), "GBs": round(dbytes / (d_us * 1e-6) / 1e9, 1),
                            "bytes": dbytes, "note": "absmax input of 2.8 MB (a warm-cache size by nature)"},
           "quantize_dq_fused": {"median_us": round(f_us, 2),
                                 "GBs": round((4 * n + n // 2 + nb + 4 * ((nb + 255) // 256)) / (f_us * 1e-6) / 1e9, 1),
                                 "frac_hbm": round((4 * n + n // 2 + nb + 4 * ((nb + 255) // 256)) / (f_us * 1e-6)
                                                   / 1e9 / PEAK_HBM_GBS, 4),
                                 "bytes": 4 * n + n // 2 + nb + 4 * ((nb + 255) // 256)},
           "quantize_dq_fused_other_types": types}
    srcs = [x.to(torch.bfloat16) for x in srcs]
    torch.cuda.empty_cache()
    for x in srcs:
        qlora.quantize_nf4(x, codes, absmax)
    b_us = _event_median(torch, lambda x: qlora.quantize_nf4(x, codes, absmax), srcs, reps)
    bbytes = 2 * n + n // 2 + 4 * nb
    res["quantize_bf16"] = {"median_us": round(b_us, 2), "GBs": round(bbytes / (b_us * 1e-6) / 1e9, 1),
                            "frac_hbm": round(bbytes / (b_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "bytes": bbytes}
    del srcs
    torch.cuda.empty_cache()
    return res


def bench_optimizer(torch, qlora, synth):
    """AdamW with global-norm clipping over the adapters of the whole 65B set
    (r = 64 on all 560 linears: 800 M parameters in one flat buffer), state
    in HBM; and the paged mode (state in pinned host memory) on one layer's
    adapters.  Median of 5 event-timed steps each."""
    wl = synth.WORKLOADS["full65b"]
    res = {}
    for label, layers, paged in (("device_state", wl.layers, False), ("paged_state", 1, True)):
        n = sum(wl.r * (l.K + l.N) for l in wl.linears) * layers
        g = torch.Generator(device="cuda")
        g.manual_seed(7)
        param = (torch.randn(n, generator=g, device="cuda") * 0.01).to(torch.bfloat16)
        grad = torch.randn(n, generator=g, device="cuda").to(torch.bfloat16)
        master = param.float()
        m = torch.zeros(n, device="cuda")
        v = torch.zeros(n, device="cuda")
        if paged:
            master, m, v = (x.cpu().pin_memory() for x in (master, m, v))
        ws = torch.empty(max(1, qlora.adamw_workspace_bytes(n)), dtype=torch.uint8, device="cuda")
        steps = iter(range(1, 100))
        qlora.adamw_step(param, master, m, v, grad, next(steps), 1e-4, max_grad_norm=1.0, workspace=ws)
        us = _event_median(torch, lambda _: qlora.adamw_step(param, master, m, v, grad, next(steps), 1e-4,
                                                              max_grad_norm=1.0, workspace=ws), [0], 5)
        # grad read twice (norm, update), param written, master/m/v read and written
        nbytes = n * (2 * 2 + 2 + 3 * 8)
        res[label] = {"params": n, "median_us": round(us, 1), "GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "bytes": nbytes}
        if not paged:
            res[label]["frac_hbm"] = round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        else:
            res[label]["note"] = "master, m, v (24 B/param) cross the host link each step"
        del param, grad, master, m, v, ws
        torch.cuda.empty_cache()
    res["workload"] = "AdamW + global-norm clipping over the LoRA adapters (r=64) of the 65B set"
    return res


def measure_peaks(torch):
    """The copy bandwidth and bf16 MFMA rate this GPU sustains (probes in
    bench_peaks.so), medians of 5 event-timed launches."""
    path = os.path.join(ROOT, "bench_peaks.so")
    if not os.path.exists(path):
        return None
    P = ctypes.CDLL(path)
    P.qlora_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.qlora_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    blocks, iters = 1024, 20000
    for _ in range(2):
        P.qlora_peak_mfma(blocks, iters, ctypes.c_void_p(out.data_ptr()), st)
    us = _event_median(torch, lambda _: P.qlora_peak_mfma(blocks, iters, ctypes.c_void_p(out.data_ptr()), st),
                       [0], 5)
    mfma = blocks * 4 * iters * 8 * 32 * 32 * 16 * 2 / (us * 1e-6) / 1e12
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        P.qlora_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, 8192, st)
    cus = _event_median(torch, lambda _: P.qlora_peak_copy(ctypes.c_void_p(src.data_ptr()),
                                                            ctypes.c_void_p(dst.data_ptr()), nbytes, 8192, st),
                        [0], 5)
    copy = 2 * nbytes / (cus * 1e-6) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"mfma_bf16_TFLOPs": round(mfma, 1), "mfma_frac_of_spec": round(mfma / PEAK_BF16_TFLOPS, 4),
            "copy_GBs": round(copy, 1), "copy_frac_of_spec": round(copy / PEAK_HBM_GBS, 4),
            "probes": "v_mfma_f32_32x32x16_bf16 chains, 4 waves per SIMD; 2 GiB device copy (read + write)"}


def dense_gemm_reference(torch, T=512):
    """Context for the GEMM rate: the same 14 GEMMs of one 65B layer (the
    forward X W^T and the dX dY W of q, k, v, o, gate, up, down at 512
    tokens) as dense bf16 torch.matmul (the platform BLAS), with no 4-bit
    decode and no adapter term; two weight copies per shape, medians of 5
    event-timed passes."""
    shapes = [(8192, 8192)] * 4 + [(22016, 8192)] * 2 + [(8192, 22016)]
    total_us, flops, per = 0.0, 0, {}
    for (N, K) in sorted(set(shapes)):
        ws = [torch.randn(N, K, device="cuda", dtype=torch.bfloat16) for _ in range(2)]
        x = torch.randn(T, K, device="cuda", dtype=torch.bfloat16)
        dy = torch.randn(T, N, device="cuda", dtype=torch.bfloat16)
        for w in ws:
            torch.matmul(x, w.t())
            torch.matmul(dy, w)
        fwd = _event_median(torch, lambda i: torch.matmul(x, ws[i % 2].t()), [0, 1], 5)
        dx = _event_median(torch, lambda i: torch.matmul(dy, ws[i % 2]), [0, 1], 5)
        n = shapes.count((N, K))
        total_us += n * (fwd + dx)
        flops += n * 2 * 2 * T * N * K
        per[f"{N}x{K}"] = {"fwd_us": round(fwd, 1), "dx_us": round(dx, 1),
                           "fwd_TFLOPs": round(2 * T * N * K / (fwd * 1e-6) / 1e12, 1),
                           "dx_TFLOPs": round(2 * T * N * K / (dx * 1e-6) / 1e12, 1)}
        del ws, x, dy
        torch.cuda.empty_cache()
    rate = flops / (total_us * 1e-6) / 1e12
    return {"workload": "dense bf16 torch.matmul of one 65B layer's forward and dX GEMMs at T=512 "
                        "(no NF4 decode, no adapter)", "TFLOPs": round(rate, 1),
            "frac_of_spec": round(rate / PEAK_BF16_TFLOPS, 4), "per_shape": per}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, untouched, on a bounded sample.
# ---------------------------------------------------------------------------
def cpu_baseline(synth):
    """The oracle timed per stage on one linear of the 65B set (q_proj,
    8192 x 8192, 512 tokens, r=64): quantize + double quant of a 2048-row
    slice of its weight, fp64 dequantize, forward, backward; median of 3 each.
    The whole-set figures are extrapolated by flops and parameter count."""
    import numpy as np
    from oracle import lora, nf4
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:
        threadpool_info = threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    blas = cores
    if threadpool_info is not None:
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            blas = max(p.get("num_threads", cores) for p in info)
    T, N, K, r, alpha = 512, 8192, 8192, 64, 16.0
    rows = 2048
    W = synth.weight(N, K, 0)
    Wq = W[:rows]

    def med3(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return median(ts)

    t_quant = med3(lambda: nf4.quantize_nf4(Wq))
    codes, absmax = nf4.quantize_nf4(Wq)
    t_dq = med3(lambda: nf4.double_quant(absmax))
    t_quant_1t = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t_quant_1t = med3(lambda: nf4.quantize_nf4(Wq))
    codes, q8, s2, _ = nf4.quantize_all(W)
    del W
    t_deq = med3(lambda: nf4.dequantize(codes, q8, s2, N * K, "bf16"))
    Wd = nf4.dequantize(codes, q8, s2, N * K, "bf16").reshape(N, K)
    X = nf4.bf16_bits_to_f32(synth.x_bits(T, K, 0))
    A = nf4.bf16_bits_to_f32(synth.a_bits(K, r, 0))
    B = nf4.bf16_bits_to_f32(synth.b_bits(r, N, 0))
    dY = nf4.bf16_bits_to_f32(synth.dy_bits(T, N, 0))
    t_fwd = med3(lambda: lora.linear_fwd(X, Wd, A, B, alpha, r))
    t_bwd = med3(lambda: lora.linear_bwd(dY, X, Wd, A, B, alpha, r))
    fl = fwdbwd_flops(T, N, K, r)
    value = fl / (t_fwd + t_bwd) / 1e12
    qparams = rows * K
    wl = synth.WORKLOADS["full65b"]
    set_flops = sum(fwdbwd_flops(wl.T, l.N, l.K, wl.r) for l in wl.linears) * wl.layers
    set_params = sum(l.N * l.K for l in wl.linears) * wl.layers
    return {"value": round(value, 6), "unit": "TFLOP/s", "cores": int(blas), "kind": "oracle",
            "sample": f"one 65B q_proj linear (8192x8192, T=512, r=64): fp64 forward + backward, median of 3; "
                      f"quantize + double quant on a {rows}x{K} slice",
            "host_cpus": cores, "blas_threads": int(blas),
            "stages_s": {"quantize": round(t_quant, 4), "quantize_1thread": None if t_quant_1t is None
                         else round(t_quant_1t, 4), "double_quant": round(t_dq, 4),
                         "dequantize_fp64": round(t_deq, 4), "forward": round(t_fwd, 4),
                         "backward": round(t_bwd, 4)},
            "quantize_GBs": round(4.5625 * qparams / t_quant / 1e9, 4),
            "quantize_GBs_1thread": None if t_quant_1t is None else round(4.5625 * qparams / t_quant_1t / 1e9, 4),
            "extrapolated_full65b": {"fwd_bwd_s_per_step": round(set_flops / (value * 1e12), 1),
                                     "quantize_all_s": round(set_params / qparams * (t_quant + t_dq), 1),
                                     "label": "extrapolated from the one-linear sample by flops and parameters"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="full65b", choices=["full65b", "layer33b", "mlp7b", "tiny"])
    ap.add_argument("--no-extras", action="store_true",
                    help="headline workload only (no other workloads, GEMV, quantize or peak probes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default="workloads,gemv,gemv_grouped,quantize,optimizer,peaks",
                    help="extra legs to run after the headline (comma list)")
    ap.add_argument("--skip-headline", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this layer is measured on one GPU only "
              "(the library has no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_nf4_quantized_21_amd import qlora, synth
    qlora.lib()
    torch.cuda.set_device(0)

    out = {"metric": METRIC}
    legs = set(args.legs.split(",")) if not args.no_extras else set()
    value = None
    if not args.skip_headline:
        print(f"bench: {args.workload} set-up", file=sys.stderr, flush=True)
        head = bench_workload(torch, qlora, synth, args.workload, args.steps, args.warmup)
        value = head["value"]
        out.update({
            "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": head["workload"] + " (NF4 + double quant base resident in HBM, LoRA fwd+bwd on "
                                   "every linear)",
                       "tokens": head["tokens"], "r": head["r"], "alpha": head["alpha"], "layers": head["layers"],
                       "linears": head["linears"], "parallelism": "single GPU",
                       "flop_per_step": head["flop_per_step"]},
            "frac_of_bf16_peak": head["frac_of_bf16_peak"],
            "roofline": head["roofline"],
            "kernels": head["kernels"],
            "quantize_all": head["quantize_all"],
        })
        print(f"bench: {args.workload} {value} TFLOP/s", file=sys.stderr, flush=True)
    if "workloads" in legs:
        out["workloads"] = {}
        for key in ("layer33b", "mlp7b"):
            if key == args.workload:
                continue
            print(f"bench: {key}", file=sys.stderr, flush=True)
            res = bench_workload(torch, qlora, synth, key, 10 if key == "layer33b" else 20, 3)
            res.pop("kernels")
            out["workloads"][key] = res
    if "gemv" in legs:
        print("bench: gemv", file=sys.stderr, flush=True)
        out["gemv"] = bench_gemv(torch, qlora, synth)
    if "gemv_grouped" in legs:
        print("bench: gemv grouped", file=sys.stderr, flush=True)
        out["gemv_grouped"] = bench_gemv_grouped(torch, qlora, synth)
    if "quantize" in legs:
        print("bench: quantize", file=sys.stderr, flush=True)
        out["quantize"] = bench_quantize(torch, qlora)
    if "optimizer" in legs:
        print("bench: optimizer", file=sys.stderr, flush=True)
        out["optimizer"] = bench_optimizer(torch, qlora, synth)
        if "ms_per_step" in out:
            out["optimizer"]["headline_step_with_optimizer_ms"] = round(
                out["ms_per_step"] + out["optimizer"]["device_state"]["median_us"] / 1e3, 3)
    if "peaks" in legs:
        print("bench: peaks", file=sys.stderr, flush=True)
        peaks = measure_peaks(torch)
        if peaks is not None and value is not None:
            peaks["headline_frac_of_measured_mfma"] = round(value / peaks["mfma_bf16_TFLOPs"], 4)
            if out.get("roofline"):
                peaks["roofline_frac_of_measured_mfma"] = round(out["roofline"]["achieved"] /
                                                               peaks["mfma_bf16_TFLOPs"], 4)
        if peaks is not None:
            for leg in ("gemv", "gemv_grouped"):
                if leg in out:
                    peaks[f"{leg}_frac_of_measured_copy"] = round(out[leg]["value"] / peaks["copy_GBs"], 4)
        if peaks is not None:
            peaks["dense_bf16_gemm_reference"] = dense_gemm_reference(torch)
        out["peaks"] = peaks
    if not args.no_cpu_baseline:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
