"""Workload and summariser for rocprofv3 measurements of the NF4 linear kernels.

`run` launches, on cuda:0, a few fwd+bwd steps of a workload's linears (by
default two layers of the LLaMA-65B-shaped set: q/k/v/o 8192x8192, gate/up
8192->22016, down 22016->8192, 512 tokens, LoRA r=64; every layer has the
same shapes, so per-launch figures are those of the 80-layer set), a few
small-token forwards (4096x4096, 4 tokens), and a plain copy of a known
number of bytes that calibrates the HBM byte counters:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o fetch -- \
        python profile_run.py run
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o write -- \
        python profile_run.py run

`traffic` turns the two counter CSVs into per-kernel HBM bytes per launch,
scaled by what the same counters read for the copy, and writes
profiles/traffic_<kernel>_<workload>.json (with a hash of the kernel sources
it was measured on) and a readable profiles/traffic_<workload>.md.

`stats` turns a `rocprofv3 --kernel-trace --stats --output-format csv` kernel
statistics file into a short markdown table.

`mfma` summarises a third counter pass,

    rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --output-format csv -d OUT/mfma -o mfma -- \
        python profile_run.py run

into profiles/mfma_<workload>.md: per kernel the share of SIMD cycles with
the matrix cores busy (MfmaUtil, percent) and the bf16 MFMA flops executed
per launch beside the algorithmic flops.
"""

from __future__ import annotations

import argparse
import csv
import dataclasses
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "bit_nf4_quantized_21_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_BYTES = 512 << 20
R, ALPHA = 64, 16.0
GEMV = (4, 4096, 4096)

# kernel -> sources it is built from
KERNEL_SOURCES = {
    "gemm_fwd_kernel": ["gemm_fwd.hip", "gemm.hpp", "splitk.hpp", "common.hpp"],
    "gemm_dx_kernel": ["gemm_dx.hip", "gemm.hpp", "splitk.hpp", "common.hpp"],
    "tokdot_partial_kernel": ["lora.hip", "lora.hpp", "common.hpp"],
    "rowdot_partial_kernel": ["lora.hip", "lora.hpp", "common.hpp"],
    "gemv_fwd_kernel": ["gemv.hip", "gemm.hpp", "common.hpp"],
}


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def dq_bytes(N, K):
    nb = N * K // 64
    return N * K // 2 + nb + 4 * ((nb + 255) // 256)


def algorithmic_bytes(kernel, T, N, K, r):
    """Each operand the kernel must touch, read or written once."""
    if kernel == "gemm_fwd_kernel":
        return 2 * T * K + dq_bytes(N, K) + 2 * r * N + 4 * T * r + 2 * T * N
    if kernel == "gemm_dx_kernel":
        return 2 * T * N + dq_bytes(N, K) + 2 * K * r + 4 * T * r + 2 * T * K
    if kernel == "gemv_fwd_kernel":
        return 2 * T * K + dq_bytes(N, K) + 2 * r * N + 4 * T * r + 2 * T * N
    return None


def algorithmic_flops(kernel, T, N, K, r):
    if kernel == "gemm_fwd_kernel":
        return 2 * T * N * K + 2 * T * r * N
    if kernel == "gemm_dx_kernel":
        return 2 * T * N * K + 2 * T * r * K
    if kernel == "gemv_fwd_kernel":
        return 2 * T * N * K + 2 * T * r * N
    return None


def workload_shapes(workload):
    from bit_nf4_quantized_21_amd import synth
    wl = synth.WORKLOADS[workload]
    return wl.T, [(l.N, l.K) for l in wl.linears]


def launches_per_layer(workload):
    """GEMM launches per layer: the step batches q/k/v and gate/up."""
    import bench
    from bit_nf4_quantized_21_amd import synth
    names = [l.name for l in synth.WORKLOADS[workload].linears]
    n = 0
    for i, nm in enumerate(names):
        prev = names[i - 1] if i else None
        if not (prev and any(nm in fs and prev in fs for fs in bench.FUSED_SETS)):
            n += 1
    return n


def per_launch(values, workload, kernel):
    """Algorithmic work per launch of a GEMM (a launch covers a batch of
    linears) or of a per-linear kernel."""
    if values[0] is None:
        return None
    if kernel in ("gemm_fwd_kernel", "gemm_dx_kernel"):
        return sum(values) / launches_per_layer(workload)
    return sum(values) / len(values)


def run(workload, layers, steps):
    import torch
    import bench
    from bit_nf4_quantized_21_amd import qlora, synth
    qlora.lib()
    wl = synth.WORKLOADS[workload]
    wl = dataclasses.replace(wl, layers=min(layers, wl.layers))
    lins = bench.linear_list(wl)
    weights, _ = bench.quantize_all(torch, qlora, synth, wl, lins)
    Ls, groups = bench.make_linears(torch, qlora, synth, wl, lins, weights)
    del weights
    for _ in range(steps):
        for g in groups:
            bench.run_group_fwd(qlora, g, wl.alpha)
        for g in reversed(groups):
            bench.run_group_bwd(qlora, g, wl.alpha)
    torch.cuda.synchronize()
    del Ls, groups
    T, N, K = GEMV
    inp = synth.device_inputs(T, N, K, R, 0, backward=False)
    codes, absmax = qlora.quantize_nf4(inp["W"].view(-1))
    q8, s2 = qlora.double_quant(absmax)
    for _ in range(steps):
        qlora.linear_fwd(inp["X"], codes, q8, s2, inp["A"], inp["B"], ALPHA, N)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("profile_run done", flush=True)


def short_name(name):
    n = name.replace("(anonymous namespace)::", "").strip()
    if n.startswith("void "):
        n = n[5:]
    cut = min([i for i in (n.find("("), n.find("<")) if i >= 0] or [len(n)])
    return n[:cut].split("::")[-1]


def read_counter(d, counter):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    rows.append((row["Kernel_Name"], int(row["Grid_Size"]), float(row["Counter_Value"])))
    return rows


def copy_factor(rows):
    """Counter KiB per true KiB for the copy of COPY_BYTES."""
    vals = [v for (k, g, v) in rows if "copy" in k.lower() and v > 0.5 * COPY_BYTES / 1024]
    if not vals:
        raise SystemExit("copy kernel not found in counters")
    return (sum(vals) / len(vals)) / (COPY_BYTES / 1024)


def traffic(fetch_dir, write_dir, command, workload):
    fr, wr = read_counter(fetch_dir, "FETCH_SIZE"), read_counter(write_dir, "WRITE_SIZE")
    ff, wf = copy_factor(fr), copy_factor(wr)
    os.makedirs(PROFILES, exist_ok=True)
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (from the repository root):", "", "```", command, "```", "",
             f"Counter scale from a plain {COPY_BYTES >> 20} MiB device copy: FETCH_SIZE reads "
             f"{ff:.4f}x, WRITE_SIZE {wf:.4f}x the true bytes; the figures below are divided by these.", "",
             "| kernel | workload | launches | fetch MB | write MB | total MB/launch | algorithmic MB/launch | ratio |",
             "|---|---|---|---|---|---|---|---|"]
    T_w, shapes = workload_shapes(workload)
    for kernel, sources in KERNEL_SOURCES.items():
        wl = "gemv7b" if kernel == "gemv_fwd_kernel" else workload
        f = [v for (k, g, v) in fr if short_name(k) == kernel]
        w = [v for (k, g, v) in wr if short_name(k) == kernel]
        if not f or not w:
            continue
        fb = sum(f) / len(f) * 1024 / ff
        wb = sum(w) / len(w) * 1024 / wf
        if wl == workload:
            alg_b = per_launch([algorithmic_bytes(kernel, T_w, N, K, R) for (N, K) in shapes], workload, kernel)
        else:
            alg_b = algorithmic_bytes(kernel, *GEMV, R)
        rec = {"kernel": kernel, "workload": wl, "launches": len(f), "fetch_bytes_per_launch": round(fb),
               "write_bytes_per_launch": round(wb), "bytes_per_launch": round(fb + wb),
               "algorithmic_bytes_per_launch": alg_b, "copy_factor_fetch": round(ff, 5),
               "copy_factor_write": round(wf, 5), "sources": sources, "source_hash": source_hash(*sources),
               "command": command}
        with open(os.path.join(PROFILES, f"traffic_{kernel}_{wl}.json"), "w") as fo:
            json.dump(rec, fo, indent=1)
        ratio = "" if alg_b is None else f"{(fb + wb) / alg_b:.2f}"
        algs = "" if alg_b is None else f"{alg_b / 1e6:.1f}"
        lines.append(f"| {kernel} | {wl} | {len(f)} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} | "
                     f"{algs} | {ratio} |")
    with open(os.path.join(PROFILES, f"traffic_{workload}_gemv7b.md"), "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats(stats_csv, out_md, command, top=12):
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# Kernel time summary (rocprofv3 --kernel-trace --stats)", "", "Command (from the repository root):",
             "", "```", command, "```", "",
             "| kernel | calls | total ms | average us | min us | max us | share % |", "|---|---|---|---|---|---|---|"]
    for r in rows[:top]:
        lines.append(f"| {short_name(r['Name'])[:60]} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    with open(out_md, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def mfma(pmc_dir, command, workload):
    util, flops = read_counter(pmc_dir, "MfmaUtil"), read_counter(pmc_dir, "MfmaFlopsBF16")
    kernels = list(KERNEL_SOURCES) + ["xa_partial_kernel", "rowdot_reduce_kernel", "tokdot_reduce_kernel"]
    lines = ["# MFMA utilisation per kernel (rocprofv3 MfmaUtil, MfmaFlopsBF16)", "",
             "Command (from the repository root):", "", "```", command, "```", "",
             "MfmaUtil: SIMD cycles with the matrix core busy over active cycles x SIMDs, averaged over "
             "launches. Flops: bf16 MFMA flops executed per launch (padding included) beside the "
             "algorithmic flops of the workload's launches.", "",
             "| kernel | workload | launches | MfmaUtil % | MFMA GFLOP/launch | algorithmic GFLOP/launch |",
             "|---|---|---|---|---|---|"]
    for kernel in kernels:
        u = [v for (k, g, v) in util if short_name(k) == kernel]
        f = [v for (k, g, v) in flops if short_name(k) == kernel]
        if not u:
            continue
        wl = "gemv7b" if ("gemv" in kernel or "xa_" in kernel) else workload
        T_w, shapes = workload_shapes(workload)
        if wl == workload:
            alg = per_launch([algorithmic_flops(kernel, T_w, N, K, R) for (N, K) in shapes], workload, kernel)
        else:
            alg = algorithmic_flops(kernel, *GEMV, R)
        algs = "" if alg is None else f"{alg / 1e9:.1f}"
        fs = f"{sum(f) / len(f) / 1e9:.1f}" if f else ""
        lines.append(f"| {kernel} | {wl} | {len(u)} | {sum(u) / len(u):.1f} | {fs} | {algs} |")
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"mfma_{workload}_gemv7b.md"), "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--steps", type=int, default=2)
    r.add_argument("--workload", default="full65b")
    r.add_argument("--layers", type=int, default=2)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--command", required=True)
    t.add_argument("--workload", default="full65b")
    m = sub.add_parser("mfma")
    m.add_argument("pmc_dir")
    m.add_argument("--command", required=True)
    m.add_argument("--workload", default="full65b")
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("out_md")
    s.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.cmd == "run":
        run(a.workload, a.layers, a.steps)
    elif a.cmd == "traffic":
        traffic(a.fetch_dir, a.write_dir, a.command, a.workload)
    elif a.cmd == "mfma":
        mfma(a.pmc_dir, a.command, a.workload)
    else:
        stats(a.stats_csv, a.out_md, a.command)


if __name__ == "__main__":
    sys.exit(main())
