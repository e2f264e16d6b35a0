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

class LinearDesc(ctypes.Structure):
    """qlora_linear_desc: one linear of a grouped forward (device pointers)."""
    _fields_ = [("X", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("q8", ctypes.c_void_p),
                ("s2", ctypes.c_void_p), ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("XA", ctypes.c_void_p), ("K", ctypes.c_int64), ("N", ctypes.c_int64)]


class LinearBwdDesc(ctypes.Structure):
    """qlora_linear_bwd_desc: one linear of a grouped backward (device pointers)."""
    _fields_ = [("dY", ctypes.c_void_p), ("X", ctypes.c_void_p), ("XA", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("q8", ctypes.c_void_p), ("s2", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("dX", ctypes.c_void_p), ("dA", ctypes.c_void_p),
                ("dB", ctypes.c_void_p), ("K", ctypes.c_int64), ("N", ctypes.c_int64)]


_SIGNATURES = {
    "qlora_quantize_nf4": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "qlora_quantize_nf4_bf16": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "qlora_double_quant": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_p, _c_p, _c_p]),
    "qlora_dequantize_nf4": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i32, _c_p, _c_p]),
    "qlora_linear_fwd_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i32]),
    "qlora_linear_bwd_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i32]),
    "qlora_linear_fwd": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_f,
                                        _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "qlora_linear_fwd_noalloc": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32,
                                                _c_f, _c_p, _c_p, _c_p]),
    "qlora_linear_bwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p,
                                        _c_i32, _c_f, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "qlora_4bit_table": (ctypes.c_int, [_c_i32, ctypes.POINTER(ctypes.c_float)]),
    "qlora_quantize_4bit": (ctypes.c_int, [_c_p, _c_i32, _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p]),
    "qlora_quantize_dq": (ctypes.c_int, [_c_p, _c_i32, _c_i64, _c_i32, _c_p, _c_p, _c_p, _c_p]),
    "qlora_dequantize_4bit": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_p]),
    "qlora_linear_fwd_4bit": (ctypes.c_int, [_c_i32, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32,
                                             _c_f, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "qlora_linear_bwd_4bit": (ctypes.c_int, [_c_i32, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p,
                                             _c_p, _c_i32, _c_f, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "qlora_save_4bit": (ctypes.c_int, [ctypes.c_char_p, _c_i32, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "qlora_load_4bit_info": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i64),
                                            ctypes.POINTER(_c_i64)]),
    "qlora_load_4bit": (ctypes.c_int, [ctypes.c_char_p, _c_i32, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "qlora_linear_fwd_grouped_workspace_bytes": (_c_sz, [_c_i32, ctypes.POINTER(LinearDesc), _c_i64, _c_i32]),
    "qlora_linear_fwd_grouped": (ctypes.c_int, [_c_i32, _c_i32, ctypes.POINTER(LinearDesc), _c_i64, _c_i32, _c_f,
                                                _c_p, _c_sz, _c_p]),
    "qlora_linear_bwd_grouped_workspace_bytes": (_c_sz, [_c_i32, ctypes.POINTER(LinearBwdDesc), _c_i64, _c_i32]),
    "qlora_linear_bwd_grouped": (ctypes.c_int, [_c_i32, _c_i32, ctypes.POINTER(LinearBwdDesc), _c_i64, _c_i32,
                                                _c_f, _c_p, _c_sz, _c_p]),
    "qlora_adamw_workspace_bytes": (_c_sz, [_c_i64]),
    "qlora_adamw_step": (ctypes.c_int, [_c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_f, _c_f, _c_f, _c_f, _c_f,
                                        _c_f, _c_p, _c_p, _c_sz, _c_p]),
    "qlora_timing_enable": (None, [ctypes.c_int]),
    "qlora_timing_read": (ctypes.c_int, [ctypes.c_char_p, _c_sz]),
    "qlora_nf4_codebook": (None, [ctypes.POINTER(ctypes.c_float)]),
    "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_last_hip_error": (ctypes.c_int, []),
    "qlora_device_status": (ctypes.c_int, [_c_p]),
}


QTYPES = {"nf4": 0, "int4": 1, "fp4": 2}


def _qtype(qtype):
    if qtype not in QTYPES:
        raise ValueError(f"qtype must be one of {sorted(QTYPES)}")
    return QTYPES[qtype]


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


def _need(t, n, name):
    """The caller's buffer must hold at least n elements (a short buffer would
    be written past its end by the kernels)."""
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, {n} needed")
    return t


def _weight(codes, q8, s2, N, K):
    nb = N * K // 64
    _need(codes, N * K // 2, "codes")
    _need(q8, nb, "q8")
    _need(s2, (nb + 255) // 256, "s2")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def device_status(stream=None):
    """Raise QLoRAError if a kernel's bounded wait ran out since the last
    query (waits for the stream; clears the status)."""
    _check(lib().qlora_device_status(_stream(stream)))


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


def table_4bit(qtype="nf4"):
    """The library's 16 fp32 decode values of a stored 4-bit type, by code."""
    buf = (ctypes.c_float * 16)()
    _check(lib().qlora_4bit_table(_qtype(qtype), buf))
    return [buf[i] for i in range(16)]


def quantize_nf4(W, codes=None, absmax=None, stream=None, qtype="nf4"):
    """W: fp32 or bf16 CUDA tensor (flattened row-major).  Returns (codes u8,
    absmax f32).  qtype selects the stored 4-bit type (nf4, int4, fp4)."""
    torch = _torch()
    bf16 = W.dtype == torch.bfloat16
    _dev(W, torch.bfloat16 if bf16 else torch.float32, "W")
    n = W.numel()
    nb = (n + 63) // 64
    codes = torch.empty(n // 2, dtype=torch.uint8, device=W.device) if codes is None else codes
    absmax = torch.empty(nb, dtype=torch.float32, device=W.device) if absmax is None else absmax
    _need(_dev(codes, torch.uint8, "codes"), n // 2, "codes")
    _need(_dev(absmax, torch.float32, "absmax"), nb, "absmax")
    _check(lib().qlora_quantize_4bit(_p(W), 1 if bf16 else 0, n, 64, _qtype(qtype), _p(codes), _p(absmax),
                                     _stream(stream)))
    return codes, absmax


def quantize_dq(W, qtype="nf4", codes=None, q8=None, s2=None, stream=None):
    """Quantization and double quantization in one pass.  Returns (codes u8,
    q8 u8, s2 f32), bit-identical to quantize_nf4 followed by double_quant."""
    torch = _torch()
    bf16 = W.dtype == torch.bfloat16
    _dev(W, torch.bfloat16 if bf16 else torch.float32, "W")
    n = W.numel()
    nb = (n + 63) // 64
    ng = (nb + 255) // 256
    codes = torch.empty(n // 2, dtype=torch.uint8, device=W.device) if codes is None else codes
    q8 = torch.empty(nb, dtype=torch.uint8, device=W.device) if q8 is None else q8
    s2 = torch.empty(ng, dtype=torch.float32, device=W.device) if s2 is None else s2
    _need(_dev(codes, torch.uint8, "codes"), n // 2, "codes")
    _need(_dev(q8, torch.uint8, "q8"), nb, "q8")
    _need(_dev(s2, torch.float32, "s2"), ng, "s2")
    _check(lib().qlora_quantize_dq(_p(W), 1 if bf16 else 0, n, _qtype(qtype), _p(codes), _p(q8), _p(s2),
                                   _stream(stream)))
    return codes, q8, s2


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


def dequantize_nf4(codes, q8, s2, n, dtype=None, out=None, stream=None, qtype="nf4"):
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
    _need(codes, n // 2, "codes")
    _need(q8, (n + 63) // 64, "q8")
    _need(s2, ((n + 63) // 64 + 255) // 256, "s2")
    _need(out, n, "out")
    _check(lib().qlora_dequantize_4bit(_p(codes), _p(q8), _p(s2), n, _qtype(qtype),
                                       1 if dtype == torch.bfloat16 else 0, _p(out), _stream(stream)))
    return out


def linear_fwd_workspace_bytes(T, K, N, r):
    return int(lib().qlora_linear_fwd_workspace_bytes(T, K, N, r))


def linear_bwd_workspace_bytes(T, K, N, r):
    return int(lib().qlora_linear_bwd_workspace_bytes(T, K, N, r))


def _workspace(nbytes, device, ws):
    """The caller's workspace if given (the library checks its size), else a
    new one of the size the library asks for."""
    torch = _torch()
    if ws is not None:
        _dev(ws, torch.uint8, "workspace")
        if ws.numel() < nbytes:
            raise ValueError(f"workspace holds {ws.numel()} bytes, {nbytes} needed")
        return ws
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def linear_fwd(X, codes, q8, s2, A, B, alpha, N, Y=None, XA=None, workspace=None, stream=None, qtype="nf4"):
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
    _weight(codes, q8, s2, N, K)
    Y = torch.empty(T, N, dtype=torch.bfloat16, device=X.device) if Y is None else Y
    XA = torch.empty(T, r, dtype=torch.float32, device=X.device) if XA is None else XA
    _need(_dev(Y, torch.bfloat16, "Y"), T * N, "Y")
    _need(_dev(XA, torch.float32, "XA"), T * r, "XA")
    nbytes = linear_fwd_workspace_bytes(T, K, N, r)
    workspace = _workspace(nbytes, X.device, workspace)
    _check(lib().qlora_linear_fwd_4bit(_qtype(qtype), _p(X), T, K, N, _p(codes), _p(q8), _p(s2), _p(A), _p(B), r,
                                       float(alpha), _p(Y), _p(XA), _p(workspace), nbytes, _stream(stream)))
    return Y, XA


def linear_fwd_noalloc(X, codes, q8, s2, A, B, alpha, N, Y, XA, stream=None):
    """linear_fwd with the library's static scratch as workspace: allocates
    nothing (Y and XA are the caller's).  Calls on one GPU must not overlap."""
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
    _weight(codes, q8, s2, N, K)
    _need(_dev(Y, torch.bfloat16, "Y"), T * N, "Y")
    _need(_dev(XA, torch.float32, "XA"), T * r, "XA")
    _check(lib().qlora_linear_fwd_noalloc(_p(X), T, K, N, _p(codes), _p(q8), _p(s2), _p(A), _p(B), r, float(alpha),
                                          _p(Y), _p(XA), _stream(stream)))
    return Y, XA


def grouped_workspace_bytes(shapes, T, r, backward=False):
    """Workspace bytes of a grouped forward (or backward) over linears of the
    given (K, N) shapes."""
    n = len(shapes)
    if backward:
        descs = (LinearBwdDesc * max(1, n))()
        for i, (K, N) in enumerate(shapes):
            descs[i].K, descs[i].N = K, N
        return int(lib().qlora_linear_bwd_grouped_workspace_bytes(n, descs, T, r))
    descs = (LinearDesc * max(1, n))()
    for i, (K, N) in enumerate(shapes):
        descs[i].K, descs[i].N = K, N
    return int(lib().qlora_linear_fwd_grouped_workspace_bytes(n, descs, T, r))


def linear_fwd_grouped(layers, alpha, T, r, workspace=None, stream=None, qtype="nf4"):
    """Grouped forward of several linears that share T, r and alpha.

    layers: list of dicts with X [T,K] bf16, codes, q8, s2, A [K,r], B [r,N]
    and optionally Y [T,N] bf16 and XA [T,r] f32 (allocated when absent).
    Returns the list of (Y, XA)."""
    torch = _torch()
    descs = (LinearDesc * max(1, len(layers)))()
    outs = []
    for i, L in enumerate(layers):
        X, A, B = _dev(L["X"], torch.bfloat16, "X"), _dev(L["A"], torch.bfloat16, "A"), _dev(L["B"], torch.bfloat16, "B")
        codes, q8, s2 = L["codes"], L["q8"], L["s2"]
        _dev(codes, torch.uint8, "codes")
        _dev(q8, torch.uint8, "q8")
        _dev(s2, torch.float32, "s2")
        if X.shape[0] != T or A.shape[1] != r or B.shape[0] != r or A.shape[0] != X.shape[1]:
            raise ValueError("shape mismatch")
        K, N = X.shape[1], B.shape[1]
        _weight(codes, q8, s2, N, K)
        Y = L.get("Y")
        XA = L.get("XA")
        Y = torch.empty(T, N, dtype=torch.bfloat16, device=X.device) if Y is None else Y
        XA = torch.empty(T, r, dtype=torch.float32, device=X.device) if XA is None else XA
        _need(_dev(Y, torch.bfloat16, "Y"), T * N, "Y")
        _need(_dev(XA, torch.float32, "XA"), T * r, "XA")
        descs[i] = LinearDesc(X.data_ptr(), codes.data_ptr(), q8.data_ptr(), s2.data_ptr(), A.data_ptr(),
                              B.data_ptr(), Y.data_ptr(), XA.data_ptr(), K, N)
        outs.append((Y, XA))
    n = len(layers)
    nbytes = int(lib().qlora_linear_fwd_grouped_workspace_bytes(n, descs, T, r))
    dev = layers[0]["X"].device if layers else "cuda"
    workspace = _workspace(nbytes, dev, workspace)
    _check(lib().qlora_linear_fwd_grouped(_qtype(qtype), n, descs, T, r, float(alpha), _p(workspace), nbytes,
                                          _stream(stream)))
    return outs


def linear_bwd_grouped(layers, alpha, T, r, workspace=None, stream=None, qtype="nf4"):
    """Grouped backward of several linears that share T, r and alpha.

    layers: list of dicts with dY [T,N], X [T,K], XA [T,r] (from the
    forward), codes, q8, s2, A [K,r], B [r,N], and optionally dX, dA, dB
    (allocated when absent).  Returns the list of (dX, dA, dB)."""
    torch = _torch()
    descs = (LinearBwdDesc * max(1, len(layers)))()
    outs = []
    for i, L in enumerate(layers):
        dY, X = _dev(L["dY"], torch.bfloat16, "dY"), _dev(L["X"], torch.bfloat16, "X")
        XA = _dev(L["XA"], torch.float32, "XA")
        A, B = _dev(L["A"], torch.bfloat16, "A"), _dev(L["B"], torch.bfloat16, "B")
        codes, q8, s2 = L["codes"], L["q8"], L["s2"]
        _dev(codes, torch.uint8, "codes")
        _dev(q8, torch.uint8, "q8")
        _dev(s2, torch.float32, "s2")
        K, N = X.shape[1], dY.shape[1]
        if X.shape[0] != T or dY.shape[0] != T or A.shape != (K, r) or B.shape != (r, N) or XA.shape != (T, r):
            raise ValueError("shape mismatch")
        _weight(codes, q8, s2, N, K)
        dX = L.get("dX")
        dA = L.get("dA")
        dB = L.get("dB")
        dX = torch.empty(T, K, dtype=torch.bfloat16, device=X.device) if dX is None else dX
        dA = torch.empty(K, r, dtype=torch.bfloat16, device=X.device) if dA is None else dA
        dB = torch.empty(r, N, dtype=torch.bfloat16, device=X.device) if dB is None else dB
        for t, nm, n in ((dX, "dX", T * K), (dA, "dA", K * r), (dB, "dB", r * N)):
            _need(_dev(t, torch.bfloat16, nm), n, nm)
        descs[i] = LinearBwdDesc(dY.data_ptr(), X.data_ptr(), XA.data_ptr(), codes.data_ptr(), q8.data_ptr(),
                                 s2.data_ptr(), A.data_ptr(), B.data_ptr(), dX.data_ptr(), dA.data_ptr(),
                                 dB.data_ptr(), K, N)
        outs.append((dX, dA, dB))
    n = len(layers)
    nbytes = int(lib().qlora_linear_bwd_grouped_workspace_bytes(n, descs, T, r))
    dev = layers[0]["X"].device if layers else "cuda"
    workspace = _workspace(nbytes, dev, workspace)
    _check(lib().qlora_linear_bwd_grouped(_qtype(qtype), n, descs, T, r, float(alpha), _p(workspace), nbytes,
                                          _stream(stream)))
    return outs


def linear_bwd(dY, X, XA, codes, q8, s2, A, B, alpha, dX=None, dA=None, dB=None, workspace=None, stream=None,
               qtype="nf4"):
    """Returns (dX bf16 [T,K], dA bf16 [K,r], dB bf16 [r,N])."""
    torch = _torch()
    _dev(dY, torch.bfloat16, "dY")
    _dev(X, torch.bfloat16, "X")
    if XA is not None:                 # None: recomputed from X and A (gradient checkpointing)
        _dev(XA, torch.float32, "XA")
    _dev(A, torch.bfloat16, "A")
    _dev(B, torch.bfloat16, "B")
    _dev(codes, torch.uint8, "codes")
    _dev(q8, torch.uint8, "q8")
    _dev(s2, torch.float32, "s2")
    T, K = X.shape
    N = dY.shape[1]
    r = A.shape[1]
    if A.shape != (K, r) or B.shape != (r, N) or dY.shape[0] != T or (XA is not None and XA.shape != (T, r)):
        raise ValueError("shape mismatch")
    _weight(codes, q8, s2, N, K)
    dX = torch.empty(T, K, dtype=torch.bfloat16, device=X.device) if dX is None else dX
    dA = torch.empty(K, r, dtype=torch.bfloat16, device=X.device) if dA is None else dA
    dB = torch.empty(r, N, dtype=torch.bfloat16, device=X.device) if dB is None else dB
    for t, nm, n in ((dX, "dX", T * K), (dA, "dA", K * r), (dB, "dB", r * N)):
        _need(_dev(t, torch.bfloat16, nm), n, nm)
    nbytes = linear_bwd_workspace_bytes(T, K, N, r)
    workspace = _workspace(nbytes, X.device, workspace)
    _check(lib().qlora_linear_bwd_4bit(_qtype(qtype), _p(dY), _p(X), _p(XA), T, K, N, _p(codes), _p(q8), _p(s2),
                                       _p(A), _p(B), r, float(alpha), _p(dX), _p(dA), _p(dB), _p(workspace), nbytes,
                                       _stream(stream)))
    return dX, dA, dB


def save_4bit(path, codes, q8, s2, N, K, qtype="nf4", stream=None):
    """Write a quantized N x K weight to a safetensors file (host-blocking)."""
    torch = _torch()
    _dev(codes, torch.uint8, "codes")
    _dev(q8, torch.uint8, "q8")
    _dev(s2, torch.float32, "s2")
    _weight(codes, q8, s2, N, K)
    _check(lib().qlora_save_4bit(os.fsencode(path), _qtype(qtype), N, K, _p(codes), _p(q8), _p(s2),
                                 _stream(stream)))


def load_4bit_info(path):
    """(qtype name, N, K) of a saved weight."""
    q, n, k = _c_i32(), _c_i64(), _c_i64()
    _check(lib().qlora_load_4bit_info(os.fsencode(path), ctypes.byref(q), ctypes.byref(n), ctypes.byref(k)))
    name = {v: key for key, v in QTYPES.items()}[q.value]
    return name, n.value, k.value


def load_4bit(path, device="cuda", stream=None):
    """Read a saved weight into new device tensors: (codes, q8, s2, qtype, N, K)."""
    torch = _torch()
    qtype, N, K = load_4bit_info(path)
    nb = (N * K + 63) // 64
    codes = torch.empty(N * K // 2, dtype=torch.uint8, device=device)
    q8 = torch.empty(nb, dtype=torch.uint8, device=device)
    s2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device=device)
    _check(lib().qlora_load_4bit(os.fsencode(path), _qtype(qtype), N, K, _p(codes), _p(q8), _p(s2),
                                 _stream(stream)))
    return codes, q8, s2, qtype, N, K


def adamw_workspace_bytes(n):
    return int(lib().qlora_adamw_workspace_bytes(n))


def adamw_step(param, master, m, v, grad, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
               max_grad_norm=0.0, grad_norm_out=None, workspace=None, stream=None):
    """One AdamW step over flat adapter buffers (see qlora_adamw_step).

    param, grad: bf16 CUDA tensors; master, m, v: fp32 tensors on the GPU or
    in pinned host memory (paged optimizer state).  grad_norm_out: optional
    fp32 CUDA tensor of one element."""
    torch = _torch()
    n = param.numel()
    _need(_dev(param, torch.bfloat16, "param"), n, "param")
    _need(_dev(grad, torch.bfloat16, "grad"), n, "grad")
    for t, nm in ((master, "master"), (m, "m"), (v, "v")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError(f"{nm} must be a contiguous float32 tensor")
        if not t.is_cuda and not t.is_pinned():
            raise ValueError(f"{nm} must be on the GPU or in pinned host memory")
        _need(t, n, nm)
    if grad_norm_out is not None:
        _dev(grad_norm_out, torch.float32, "grad_norm_out")
    nbytes = adamw_workspace_bytes(n)
    workspace = _workspace(nbytes, param.device, workspace)
    _check(lib().qlora_adamw_step(n, _p(param), _p(master), _p(m), _p(v), _p(grad), int(step), float(lr),
                                  float(beta1), float(beta2), float(eps), float(weight_decay), float(max_grad_norm),
                                  _p(grad_norm_out), _p(workspace), nbytes, _stream(stream)))
