#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 linear hot path on one MI355X.

Step (the timed unit): forward + backward of every linear of the workload
(default: the LLaMA-7B MLP, gate/up 4096->11008 and down 11008->4096, 2048
tokens, LoRA r=64, alpha=16), on synthetic seeded inputs already resident in
HBM.  `value` is the algorithmic fwd+bwd rate, sum over linears of
4 T N K + 6 T r (K + N) flop per step, divided by the host wall time of
exactly --steps steps bracketed by device synchronisations.

Beside it, in the same JSON line:
  roofline      the dominant kernel's algorithmic rate against the MI355X peak,
                from HIP events recorded on its launch stream during the timed
                steps (the library's per-kernel timing hooks);
  gemv          the small-token forward (LLaMA-7B q_proj 4096x4096, 4 tokens,
                r=64): dequant-GEMV kernel GB/s over 40 rotating weight copies
                (> 256 MB, so every launch streams the 4-bit weights from HBM);
  quantize      blockwise NF4 quantization (fp32 and bf16 weights) + double
                quantization GB/s;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload mlp7b|layer33b|tiny]
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

PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # HBM3E
METRIC = "QLoRA NF4 linear fwd+bwd TFLOP/s and dequant-GEMV GB/s, % of MI355X roofline"


def fwd_flops(T, N, K, r):
    return 2 * T * N * K + 2 * T * r * (K + N)


def fwdbwd_flops(T, N, K, r):
    return 4 * T * N * K + 6 * T * r * (K + N)


def kernel_flops(name, T, N, K, r):
    """Algorithmic flops of one launch of the named kernel for one linear."""
    if name == "gemm_fwd_kernel":
        return 2 * T * N * K + 2 * T * r * N
    if name == "gemm_dx_kernel":
        return 2 * T * N * K + 2 * T * r * K
    return None


def gemv_kernel_bytes(T, N, K, r):
    """Algorithmic HBM bytes of one dequant-GEMV launch: codes, 8-bit and
    fp32 second-level constants, X, B, XA in and Y out, each once."""
    nb = N * K // 64
    return N * K // 2 + nb + 4 * ((nb + 255) // 256) + 2 * T * K + 2 * r * N + 4 * T * r + 2 * T * N


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


def make_layer(torch, qlora, synth, T, N, K, r, i, backward=True):
    inp = synth.device_inputs(T, N, K, r, i, backward=backward)
    codes, absmax = qlora.quantize_nf4(inp["W"].view(-1))
    q8, s2 = qlora.double_quant(absmax)
    del inp["W"], absmax
    L = dict(T=T, N=N, K=K, r=r, codes=codes, q8=q8, s2=s2, **inp)
    dev = codes.device
    L["Y"] = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    L["XA"] = torch.empty(T, r, dtype=torch.float32, device=dev)
    L["wsf"] = torch.empty(max(1, qlora.linear_fwd_workspace_bytes(T, K, N, r)), dtype=torch.uint8, device=dev)
    if backward:
        L["dX"] = torch.empty(T, K, dtype=torch.bfloat16, device=dev)
        L["dA"] = torch.empty(K, r, dtype=torch.bfloat16, device=dev)
        L["dB"] = torch.empty(r, N, dtype=torch.bfloat16, device=dev)
        L["wsb"] = torch.empty(max(1, qlora.linear_bwd_workspace_bytes(T, K, N, r)), dtype=torch.uint8, device=dev)
    return L


def run_fwd(qlora, L, alpha):
    qlora.linear_fwd(L["X"], L["codes"], L["q8"], L["s2"], L["A"], L["B"], alpha, L["N"], Y=L["Y"], XA=L["XA"],
                     workspace=L["wsf"])


def run_bwd(qlora, L, alpha):
    qlora.linear_bwd(L["dY"], L["X"], L["XA"], L["codes"], L["q8"], L["s2"], L["A"], L["B"], alpha, dX=L["dX"],
                     dA=L["dA"], dB=L["dB"], workspace=L["wsb"])


def bench_step(torch, qlora, synth, wl, steps, warmup):
    layers = [make_layer(torch, qlora, synth, wl.T, lin.N, lin.K, wl.r, i) for i, lin in enumerate(wl.linears)]

    def step():
        for L in layers:
            run_fwd(qlora, L, wl.alpha)
            run_bwd(qlora, L, wl.alpha)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Throughput: K steps with no instrumentation in the stream.
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    # Per-kernel durations: the same K steps again with a HIP event pair
    # recorded around every launch, on the stream it is launched on (the
    # events add a few microseconds between kernels, so this pass does not
    # give the throughput).
    qlora.timing_read()
    qlora.timing_enable(True)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    qlora.timing_enable(False)
    kt = qlora.timing_read()
    ms_timed = (t3 - t2) * 1e3 / steps
    flops = sum(fwdbwd_flops(L["T"], L["N"], L["K"], L["r"]) for L in layers)
    # dominant kernel: largest total time in the timed steps
    dom = max(kt.items(), key=lambda kv: kv[1][1])
    name, (launches, total_ms) = dom
    per_step_flops = [kernel_flops(name, L["T"], L["N"], L["K"], L["r"]) for L in layers]
    roof = None
    if all(f is not None for f in per_step_flops):
        alg = sum(per_step_flops) * steps
        achieved = alg / (total_ms * 1e-3) / 1e12
        roof = {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_from_profiles(name, "mlp7b"),
                "avg_launch_us": round(total_ms * 1e3 / launches, 2), "launches": launches}
    kernels = {k: {"launches": n, "avg_us": round(t * 1e3 / n, 2), "share": round(t / sum(v[1] for v in kt.values()), 4)}
               for k, (n, t) in sorted(kt.items(), key=lambda kv: -kv[1][1])}
    if roof is not None:
        roof["events_pass_ms_per_step"] = round(ms_timed, 4)
    del layers
    torch.cuda.empty_cache()
    return ms, flops, roof, kernels


def bench_gemv(torch, qlora, synth, copies=40, iters=200):
    T, N, K, r, alpha = 4, 4096, 4096, 64, 16.0
    layers = [make_layer(torch, qlora, synth, T, N, K, r, i, backward=False) for i in range(copies)]
    X = layers[0]["X"]
    for L in layers:
        L["X"] = X
    for i in range(2 * copies):
        run_fwd(qlora, layers[i % copies], alpha)
    torch.cuda.synchronize()
    qlora.timing_read()
    qlora.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(iters):
        run_fwd(qlora, layers[i % copies], alpha)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    qlora.timing_enable(False)
    kt = qlora.timing_read()
    n, total = kt["gemv_fwd_kernel"]
    us = total * 1e3 / n
    kb = gemv_kernel_bytes(T, N, K, r)
    gbs = kb / (us * 1e-6) / 1e9
    fwd_us = sum(t for (_, t) in kt.values()) * 1e3 / iters
    wall_us = (t1 - t0) * 1e6 / iters
    res = {"workload": "llama7b-q_proj-gemv-T4-r64 (4096x4096 NF4+DQ, 4 tokens, fwd)",
           "value": round(gbs, 1), "unit": "GB/s",
           "roofline": {"kernel": "gemv_fwd_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": traffic_from_profiles("gemv_fwd_kernel", "gemv7b"),
                        "avg_launch_us": round(us, 3), "bytes_per_launch": kb},
           "fwd_path_us_gpu": round(fwd_us, 3), "fwd_path_GBs_gpu": round(gemv_path_bytes(T, N, K, r) / (fwd_us * 1e-6) / 1e9, 1),
           "fwd_call_us_wall": round(wall_us, 3),
           "kernels_avg_us": {k: round(t * 1e3 / c, 3) for k, (c, t) in kt.items()},
           "weight_copies": copies}
    del layers
    torch.cuda.empty_cache()
    return res


def bench_quantize(torch, qlora, iters=10):
    N, K = 11008, 4096
    n = N * K
    srcs = []
    for i in range(2):
        g = torch.Generator(device="cuda")
        g.manual_seed(1000 + i)
        srcs.append(torch.randn(n, generator=g, device="cuda", dtype=torch.float32) * 0.02)
    codes = torch.empty(n // 2, dtype=torch.uint8, device="cuda")
    absmax = torch.empty(n // 64, dtype=torch.float32, device="cuda")
    q8 = torch.empty(n // 64, dtype=torch.uint8, device="cuda")
    s2 = torch.empty((n // 64 + 255) // 256, dtype=torch.float32, device="cuda")
    for i in range(4):
        qlora.quantize_nf4(srcs[i % 2], codes, absmax)
        qlora.double_quant(absmax, q8, s2)
    torch.cuda.synchronize()
    qlora.timing_read()
    qlora.timing_enable(True)
    for i in range(iters):
        qlora.quantize_nf4(srcs[i % 2], codes, absmax)
        qlora.double_quant(absmax, q8, s2)
    torch.cuda.synchronize()
    qlora.timing_enable(False)
    kt = qlora.timing_read()
    qn, qt = kt["quantize_nf4_kernel"]
    dn, dt = kt["double_quant_kernel"]
    qbytes = 4 * n + n // 2 + 4 * (n // 64)
    dbytes = 4 * (n // 64) + n // 64 + 4 * ((n // 64 + 255) // 256)
    q_us, d_us = qt * 1e3 / qn, dt * 1e3 / dn
    res = {"workload": "quantize 11008x4096 fp32 -> NF4 + double quant",
           "quantize": {"avg_us": round(q_us, 2), "GBs": round(qbytes / (q_us * 1e-6) / 1e9, 1),
                        "frac_hbm": round(qbytes / (q_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "bytes": qbytes},
           "double_quant": {"avg_us": round(d_us, 2), "GBs": round(dbytes / (d_us * 1e-6) / 1e9, 1), "bytes": dbytes}}
    # The same weights stored as bf16 (how pretrained checkpoints ship).
    srcs = [x.to(torch.bfloat16) for x in srcs]
    for i in range(4):
        qlora.quantize_nf4(srcs[i % 2], codes, absmax)
    torch.cuda.synchronize()
    qlora.timing_read()
    qlora.timing_enable(True)
    for i in range(iters):
        qlora.quantize_nf4(srcs[i % 2], codes, absmax)
    torch.cuda.synchronize()
    qlora.timing_enable(False)
    bn, bt = qlora.timing_read()["quantize_nf4_bf16_kernel"]
    bbytes = 2 * n + n // 2 + 4 * (n // 64)
    b_us = bt * 1e3 / bn
    res["quantize_bf16"] = {"avg_us": round(b_us, 2), "GBs": round(bbytes / (b_us * 1e-6) / 1e9, 1),
                            "frac_hbm": round(bbytes / (b_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "bytes": bbytes}
    del srcs
    torch.cuda.empty_cache()
    return res


def cpu_baseline(synth, T_sample=2048, budget_s=30.0):
    """The oracle, untuned, on the bench step itself: the three 7B MLP linears
    (gate, up, down) at T_sample tokens, r=64, each as fp64 dequantize +
    forward + backward. Quantization of W happens before the timed region.
    Linears are taken in order and the sample stops early once budget_s of
    CPU time has been spent, so a slow host still finishes in bounded time."""
    from oracle import lora, nf4
    r, alpha = 64, 16.0
    done, fl, dt = [], 0.0, 0.0
    for i, (name, N, K) in enumerate((("gate_proj", 11008, 4096), ("up_proj", 11008, 4096),
                                      ("down_proj", 4096, 11008))):
        W = synth.weight(N, K, i)
        X = nf4.bf16_bits_to_f32(synth.x_bits(T_sample, K, i))
        A = nf4.bf16_bits_to_f32(synth.a_bits(K, r, i))
        B = nf4.bf16_bits_to_f32(synth.b_bits(r, N, i))
        dY = nf4.bf16_bits_to_f32(synth.dy_bits(T_sample, N, i))
        codes, q8, s2, _ = nf4.quantize_all(W)
        del W
        t0 = time.perf_counter()
        Wd = nf4.dequantize(codes, q8, s2, N * K, "bf16").reshape(N, K)
        lora.linear_fwd(X, Wd, A, B, alpha, r)
        lora.linear_bwd(dY, X, Wd, A, B, alpha, r)
        dt += time.perf_counter() - t0
        fl += fwdbwd_flops(T_sample, N, K, r)
        done.append(name)
        del Wd, X, dY
        if dt > budget_s:
            break
    cores = len(os.sched_getaffinity(0))
    threads = cores
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            threads = max(p.get("num_threads", cores) for p in info)
    except Exception:
        pass
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{'+'.join(done)} of the 7B MLP at {T_sample} tokens, r=64: "
                      f"fp64 dequantize + fwd + bwd, {dt:.2f} s",
            "host_cpus": cores}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mlp7b", choices=["mlp7b", "layer33b", "tiny"])
    ap.add_argument("--no-extras", action="store_true", help="skip the GEMV and quantize measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    wl = synth.WORKLOADS[args.workload]

    ms, flops, roof, kernels = bench_step(torch, qlora, synth, wl, args.steps, args.warmup)
    value = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + " (NF4 + double quant base, LoRA fwd+bwd on every linear)",
                   "tokens": wl.T, "r": wl.r, "alpha": wl.alpha,
                   "linears": [[l.name, l.N, l.K] for l in wl.linears], "parallelism": "single GPU",
                   "flop_per_step": flops},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_extras:
        out["gemv"] = bench_gemv(torch, qlora, synth)
        out["quantize"] = bench_quantize(torch, qlora)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
