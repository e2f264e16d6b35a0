"""ctypes binding of libqlora (include/qlora.h).

Argument marshalling only: torch tensors on the GPU supply device pointers
and the current HIP stream; every step of the computation runs in the
library's kernels.  The library is loaded from this package directory and
must have been built (python -m bit_nf4_quantized_21_amd.build); there is no
fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqlora.so")

_lib = None

_c_i64, _c_i32, _c_p, _c_sz, _c_f = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float

_SIGNATURES = {
    "qlora_quantize_nf4": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "qlora_quantize_nf4_bf16": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "qlora_double_quant": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "qlora_dequantize_nf4": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i32, _c_p, _c_p]),
    "qlora_linear_fwd_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i32]),
    "qlora_linear_bwd_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i32]),
    "qlora_linear_fwd": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_f,
                                        _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "qlora_linear_bwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p,
                                        _c_i32, _c_f, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "qlora_timing_enable": (None, [ctypes.c_int]),
    "qlora_timing_read": (ctypes.c_int, [ctypes.c_char_p, _c_sz]),
    "qlora_nf4_codebook": (None, [ctypes.POINTER(ctypes.c_float)]),
    "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_last_hip_error": (ctypes.c_int, []),
}


def lib():
    """Load libqlora.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_nf4_quantized_21_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class QLoRAError(RuntimeError):
    pass


def _check(rc: int):
    if rc != 0:
        msg = lib().qlora_status_string(rc).decode()
        if rc == -5:
            msg += f" (hip error {lib().qlora_last_hip_error()})"
        raise QLoRAError(msg)


def _torch():
    import torch
    return torch


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def timing_enable(on=True):
    """Bracket every library kernel launch with HIP events (benchmarks only)."""
    lib().qlora_timing_enable(1 if on else 0)


def timing_read():
    """{kernel_name: (launches, total_ms)} for the launches since the last read."""
    size = 1 << 20
    buf = ctypes.create_string_buffer(size)
    rc = lib().qlora_timing_read(buf, size)   # collects and forgets in one call
    if rc < 0:
        _check(rc)
    if rc >= size:
        raise QLoRAError("timing report truncated")
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split()
        out[name] = (int(n), float(ms))
    return out


def nf4_codebook():
    """The library's 16 fp32 NF4 values (host table)."""
    buf = (ctypes.c_float * 16)()
    lib().qlora_nf4_codebook(buf)
    return [buf[i] for i in range(16)]


def quantize_nf4(W, codes=None, absmax=None, stream=None):
    """W: fp32 or bf16 CUDA tensor (flattened row-major).  Returns (codes u8, absmax f32)."""
    torch = _torch()
    bf16 = W.dtype == torch.bfloat16
    _dev(W, torch.bfloat16 if bf16 else torch.float32, "W")
    n = W.numel()
    nb = (n + 63) // 64
    codes = torch.empty(n // 2, dtype=torch.uint8, device=W.device) if codes is None else codes
    absmax = torch.empty(nb, dtype=torch.float32, device=W.device) if absmax is None else absmax
    _dev(codes, torch.uint8, "codes")
    _dev(absmax, torch.float32, "absmax")
    if codes.numel() < n // 2 or absmax.numel() < nb:
        raise ValueError("output buffers too small")
    entry = lib().qlora_quantize_nf4_bf16 if bf16 else lib().qlora_quantize_nf4
    _check(entry(_p(W), n, 64, _p(codes), _p(absmax), _stream(stream)))
    return codes, absmax


def double_quant(absmax, q8=None, s2=None, stream=None):
    """absmax: fp32 CUDA tensor [nb].  Returns (q8 u8 [nb], s2 f32 [ceil(nb/256)])."""
    torch = _torch()
    _dev(absmax, torch.float32, "absmax")
    nb = absmax.numel()
    ng = (nb + 255) // 256
    q8 = torch.empty(nb, dtype=torch.uint8, device=absmax.device) if q8 is None else q8
    s2 = torch.empty(ng, dtype=torch.float32, device=absmax.device) if s2 is None else s2
    _dev(q8, torch.uint8, "q8")
    _dev(s2, torch.float32, "s2")
    if q8.numel() < nb or s2.numel() < ng:
        raise ValueError("output buffers too small")
    _check(lib().qlora_double_quant(_p(absmax), nb, 256, _p(q8), _p(s2), _stream(stream)))
    return q8, s2


def dequantize_nf4(codes, q8, s2, n, dtype=None, out=None, stream=None):
    """Dense weight from NF4 + double-quant storage; bf16 (default) or fp32."""
    torch = _torch()
    dtype = torch.bfloat16 if dtype is None else dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("dtype must be bfloat16 or float32")
    _dev(codes, torch.uint8, "codes")
    _dev(q8, torch.uint8, "q8")
    _dev(s2, torch.float32, "s2")
    out = torch.empty(n, dtype=dtype, device=codes.device) if out is None else out
    _dev(out, dtype, "out")
    _check(lib().qlora_dequantize_nf4(_p(codes), _p(q8), _p(s2), n, 1 if dtype == torch.bfloat16 else 0,
                                      _p(out), _stream(stream)))
    return out


def linear_fwd_workspace_bytes(T, K, N, r):
    return int(lib().qlora_linear_fwd_workspace_bytes(T, K, N, r))


def linear_bwd_workspace_bytes(T, K, N, r):
    return int(lib().qlora_linear_bwd_workspace_bytes(T, K, N, r))


def _workspace(nbytes, device, ws):
    torch = _torch()
    if nbytes == 0:
        return ws
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws


def linear_fwd(X, codes, q8, s2, A, B, alpha, N, Y=None, XA=None, workspace=None, stream=None):
    """Y = X W'^T + (alpha/r) (X A) B and XA = X A.  Returns (Y bf16 [T,N], XA f32 [T,r])."""
    torch = _torch()
    _dev(X, torch.bfloat16, "X")
    _dev(A, torch.bfloat16, "A")
    _dev(B, torch.bfloat16, "B")
    _dev(codes, torch.uint8, "codes")
    _dev(q8, torch.uint8, "q8")
    _dev(s2, torch.float32, "s2")
    T, K = X.shape
    r = A.shape[1]
    if A.shape != (K, r) or B.shape != (r, N):
        raise ValueError("A must be [K,r] and B [r,N]")
    Y = torch.empty(T, N, dtype=torch.bfloat16, device=X.device) if Y is None else Y
    XA = torch.empty(T, r, dtype=torch.float32, device=X.device) if XA is None else XA
    _dev(Y, torch.bfloat16, "Y")
    _dev(XA, torch.float32, "XA")
    nbytes = linear_fwd_workspace_bytes(T, K, N, r)
    workspace = _workspace(nbytes, X.device, workspace)
    _check(lib().qlora_linear_fwd(_p(X), T, K, N, _p(codes), _p(q8), _p(s2), _p(A), _p(B), r, float(alpha),
                                  _p(Y), _p(XA), _p(workspace), nbytes, _stream(stream)))
    return Y, XA


def linear_bwd(dY, X, XA, codes, q8, s2, A, B, alpha, dX=None, dA=None, dB=None, workspace=None, stream=None):
    """Returns (dX bf16 [T,K], dA bf16 [K,r], dB bf16 [r,N])."""
    torch = _torch()
    _dev(dY, torch.bfloat16, "dY")
    _dev(X, torch.bfloat16, "X")
    _dev(XA, torch.float32, "XA")
    _dev(A, torch.bfloat16, "A")
    _dev(B, torch.bfloat16, "B")
    _dev(codes, torch.uint8, "codes")
    _dev(q8, torch.uint8, "q8")
    _dev(s2, torch.float32, "s2")
    T, K = X.shape
    N = dY.shape[1]
    r = A.shape[1]
    if A.shape != (K, r) or B.shape != (r, N) or dY.shape[0] != T or XA.shape != (T, r):
        raise ValueError("shape mismatch")
    dX = torch.empty(T, K, dtype=torch.bfloat16, device=X.device) if dX is None else dX
    dA = torch.empty(K, r, dtype=torch.bfloat16, device=X.device) if dA is None else dA
    dB = torch.empty(r, N, dtype=torch.bfloat16, device=X.device) if dB is None else dB
    for t, nm in ((dX, "dX"), (dA, "dA"), (dB, "dB")):
        _dev(t, torch.bfloat16, nm)
    nbytes = linear_bwd_workspace_bytes(T, K, N, r)
    workspace = _workspace(nbytes, X.device, workspace)
    _check(lib().qlora_linear_bwd(_p(dY), _p(X), _p(XA), T, K, N, _p(codes), _p(q8), _p(s2), _p(A), _p(B), r,
                                  float(alpha), _p(dX), _p(dA), _p(dB), _p(workspace), nbytes, _stream(stream)))
    return dX, dA, dB
