"""4-bit comparison data types (Int4, FP4) and quantization error, in fp64.
TEST INFRASTRUCTURE ONLY.

The pages state that NF4 gives better results than 4-bit integers and 4-bit
floats (news write-up, innovations list and the NF4-vs-FP4 section; project
page, core innovations).  Reading R11 fixes the comparison types:
  * Int4, symmetric absmax with the 15 levels k/7, k = -7..7 (and the 16-level
    two's-complement variant k/8, k = -8..7);
  * FP4 as E2M1 with magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} / 6 and a sign;
all with the same block of 64 and nearest rounding (ties to the lower value).
"""

from __future__ import annotations

import numpy as np

from .nf4 import BLOCK, block_absmax, codebook, quantize_all, dequantize, dequantize_fp32_absmax, quantize_nf4


def _nearest_level(u: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Nearest value of the sorted ``levels`` to each u (ties to the lower)."""
    levels = np.asarray(levels, dtype=np.float64)
    mids = (levels[:-1] + levels[1:]) / 2.0
    idx = np.searchsorted(mids, u, side="left")
    return levels[idx]


def _blockwise(w, levels, blocksize=BLOCK):
    w = np.ascontiguousarray(w, dtype=np.float64).ravel()
    a = np.repeat(block_absmax(w.astype(np.float32), blocksize).astype(np.float64), blocksize)[: w.size]
    u = np.divide(w, a, out=np.zeros_like(w), where=a > 0)
    return _nearest_level(u, levels) * a


def int4_levels(variant: str = "k7") -> np.ndarray:
    if variant == "k7":
        return np.arange(-7, 8, dtype=np.float64) / 7.0
    if variant == "k8":
        return np.arange(-8, 8, dtype=np.float64) / 8.0
    raise ValueError(variant)


def fp4_levels() -> np.ndarray:
    mag = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]) / 6.0
    return np.unique(np.concatenate([-mag, mag]))


def roundtrip(w, kind: str) -> np.ndarray:
    """Quantize-dequantize w with one of the 4-bit types; fp64 result."""
    w32 = np.ascontiguousarray(w, dtype=np.float32).ravel()
    if kind == "nf4":
        codes, absmax = quantize_nf4(w32)
        return dequantize_fp32_absmax(codes, absmax, w32.size).astype(np.float64)
    if kind == "nf4_dq":
        codes, q8, s2, _ = quantize_all(w32)
        return dequantize(codes, q8, s2, w32.size, dtype="f32").astype(np.float64)
    if kind == "int4_k7":
        return _blockwise(w32, int4_levels("k7"))
    if kind == "int4_k8":
        return _blockwise(w32, int4_levels("k8"))
    if kind == "fp4":
        return _blockwise(w32, fp4_levels())
    raise ValueError(kind)


def mse(w, kind: str) -> float:
    w64 = np.ascontiguousarray(w, dtype=np.float32).ravel().astype(np.float64)
    d = roundtrip(w, kind) - w64
    return float(np.mean(d * d))


def nf4_levels() -> np.ndarray:
    return codebook().astype(np.float64)
