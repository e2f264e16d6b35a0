"""Build tests/asan/abi_asan: the C driver linked against libqlora's objects
with the host code instrumented by AddressSanitizer (device code as usual).

    python tests/asan/build_asan.py OUT_DIR

The host sources (the C entry points, storage, timing) are compiled by hipcc
with the sanitizer flag given to the host pass only; the codebook source and
the driver by gcc/g++; the kernel sources (.hip) without the sanitizer.
"""

from __future__ import annotations

import concurrent.futures
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from bit_nf4_quantized_21_amd import build as B  # noqa: E402

SAN = ["-fsanitize=address", "-fno-omit-frame-pointer", "-g"]


def build(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    hip, hip_host, cxx = B.sources()
    jobs = []
    for f in hip:
        jobs.append([B.HIPCC, *B.HIP_FLAGS, "-c", os.path.join(B.CSRC, f), "-o", os.path.join(out_dir, f + ".o")])
    for f in hip_host:
        host_san = [a for s in SAN for a in ("-Xarch_host", s)]
        jobs.append([B.HIPCC, *B.HIP_FLAGS, *host_san, "-x", "hip", "-c", os.path.join(B.CSRC, f), "-o",
                     os.path.join(out_dir, f + ".o")])
    for f in cxx:
        jobs.append(["g++", *B.CXX_FLAGS, *SAN, "-c", os.path.join(B.CSRC, f), "-o", os.path.join(out_dir, f + ".o")])
    jobs.append(["gcc", "-O1", "-Wall", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
                 os.path.join(HERE, "abi_asan.c"), "-o", os.path.join(out_dir, "abi_asan.o")])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(B._run, jobs))
    exe = os.path.join(out_dir, "abi_asan")
    B._run([B.HIPCC, f"--offload-arch={B.ARCH}", "-fsanitize=address", "-fno-gpu-sanitize", "-o", exe,
            *[j[-1] for j in jobs]])
    return exe


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(HERE, "_build")))
