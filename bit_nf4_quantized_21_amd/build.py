"""Build libqlora.so in-tree for gfx950 with hipcc (no JIT, no cache).

    python -m bit_nf4_quantized_21_amd.build

Every HIP source is compiled with packed-FP32 instruction selection turned
off; the host-only codebook source is compiled with g++.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libqlora.so")
OBJ = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(os.path.dirname(HERE), "include")]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    return hip, ["qlora_api.cpp", "timing.cpp", "storage.cpp"], ["codebook.cpp"]


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    hip, hip_host, cxx = sources()
    jobs = []
    for f in hip + hip_host:
        o = os.path.join(OBJ, f + ".o")
        lang = [] if f.endswith(".hip") else ["-x", "hip"]
        jobs.append([HIPCC, *HIP_FLAGS, *lang, "-c", os.path.join(CSRC, f), "-o", o])
    for f in cxx:
        o = os.path.join(OBJ, f + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [j[-1] for j in jobs]
    tmp = OUT + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    return OUT


# The peak probes bench.py reads the measured MFMA and copy rates from (a
# measurement aid beside the benchmark, not part of libqlora).
PEAK_SRC = os.path.join(os.path.dirname(HERE), "bench_peaks.hip")
PEAK_OUT = os.path.join(os.path.dirname(HERE), "bench_peaks.so")


def build_peaks() -> str:
    tmp = PEAK_OUT + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", PEAK_SRC, "-o", tmp])
    os.replace(tmp, PEAK_OUT)
    return PEAK_OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_peaks())
