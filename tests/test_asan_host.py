"""Host-side memory checks of libqlora under AddressSanitizer (CPU only).

Builds tests/asan/abi_asan -- a C driver over the C entry points, linked
against libqlora's objects with the host code instrumented (the kernels are
compiled as usual) -- and runs it: argument refusals of every entry point,
workspace-size queries over many shapes, and the safetensors reader on a
valid file, every truncation, bad length fields, a header whose tensors are
far larger than the file, and seeded random corruptions of the header.  A
memory error or leak aborts the driver with the sanitizer's report.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs gcc and hipcc")
def test_host_code_under_address_sanitizer(tmp_path):
    sys.path.insert(0, os.path.join(ROOT, "tests", "asan"))
    try:
        import build_asan
    finally:
        sys.path.pop(0)
    exe = build_asan.build(str(tmp_path / "build"))
    work = tmp_path / "files"
    work.mkdir()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1")
    p = subprocess.run([exe, str(work)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=600)
    assert "AddressSanitizer" not in p.stdout and "LeakSanitizer" not in p.stdout, p.stdout[-4000:]
    assert p.returncode == 0, p.stdout[-4000:]
    assert "all host checks passed" in p.stdout
